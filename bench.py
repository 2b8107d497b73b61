"""Benchmark of one rank's tensor-parallel layer shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-7b] [--no-70b]
    python bench.py --sweep          # the 7B t=2 vs t=1 batch x prompt-length sweep

Prints ONE JSON line.  The headline step is the whole prefill hot path of
rank 0 of a 70B-shaped GQA layer split eight ways (hidden 8192, 8 of 64
query heads + 1 of 8 KV heads x 128, SwiGLU 3584 of 28672, RMSNorm, RoPE,
bf16, batch 4 x 4096 tokens, causal) -- the largest single-GPU prefill
configuration, as a layer of a stack runs it: ATTN stage (Q/K/V projection
of the normalised input with RoPE and KV-cache write, causal attention,
row-parallel output projection) -> reduce of the eight ranks' partials +
residual, fused with the MLP stage's RMSNorm -> MLP stage (gate/up
projection with SwiGLU, row-parallel down projection) -> reduce fused with
the RMSNorm of the next layer's input.  Every norm of a layer is in the
step; the first layer input's norm is made once before timing.  The other
ranks' partials are seeded stand-ins, resident in HBM before timing (they
stand for the other GPUs' contributions).

`value` is the step's algorithmic FLOPs (GEMMs + causal attention) per
second.  `roofline` covers the dominant kernel (the gate/up projection GEMM),
timed with HIP events on its launch stream inside the timed steps.
`prefill_7b` reports the same for rank 0 of a 7B-shaped layer split two ways
(hidden 4096, 16 of 32 heads, SwiGLU 5504 of 11008, batch 1 x 2048 tokens;
the other rank's partials computed by its own shard) and its
sequence-parallel variant.  `decode` / `decode_70b` report batch-1 decode of
rank 0 of the 7B layer split four ways (cache 1024) and of the 70B layer
split eight ways (cache 4096), in microseconds per token per layer, over
stacks of distinct layer copies whose weights (>= 1 GB) exceed the 256 MB
Infinity Cache.  `clock` is the GPU clock sampled while the headline steps
run, `hbm_copy_GBps` a plain device copy's rate (the measured streaming
ceiling).  `cpu_baseline` times the CPU oracle (NumPy float64) on a bounded
sample of the headline workload: one of its four sequences, whole.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard-layer prefill TFLOP/s (% MFMA peak) + decode µs/token/layer (% HBM BW)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
XGMI_LINK_GBPS = 153.0         # one xGMI link, used only by the labelled all-reduce model
ALLREDUCE_LATENCY_US = 5.0     # assumed fixed cost per all-reduce in that model
MIN_DECODE_FOOTPRINT = 1.0e9   # decode weight copies span at least this many bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-layers", type=int, default=0,
                    help="layer copies in the decode stack (0: enough for >= 1 GB of weights)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-70b", action="store_true", help="skip the 70B-shaped prefill and decode (the headline: "
                                                           "the 7B prefill takes its place)")
    ap.add_argument("--no-7b", action="store_true", help="skip the 7B-shaped prefill and decode")
    ap.add_argument("--sweep", action="store_true", help="run the 7B t=2 vs t=1 crossover sweep instead")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB three times: the known-size copy that scales rocprofv3 byte counters")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="no GPU: turn rocprofv3 outputs of this script into profiles/traffic.json and "
                         "profiles/*.md (see profiles/README.md for the commands)")
    ap.add_argument("--summarize-warmup", nargs=3, metavar=("PMC_DIR", "KEY", "OUT_MD"),
                    help="no GPU: per-dispatch duration and clock of the first dispatches of roofline kernel KEY "
                         "from a rocprofv3 --pmc GRBM_GUI_ACTIVE run, into profiles/OUT_MD")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "OUT_MD"),
                    help="no GPU: turn a rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 GRBM_GUI_ACTIVE run of this script "
                         "into profiles/OUT_MD")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work

def dims(hidden, heads, kv_heads, ffn, t):
    d = hidden // heads
    return d, heads // t, kv_heads // t, ffn // t


def prefill_flops(hidden, heads, kv_heads, ffn, t, B, S):
    """Algorithmic FLOPs of one rank's prefill step: the four projections
    plus causal attention (QK^T and PV over the causal half)."""
    d, hl, kvl, fl = dims(hidden, heads, kv_heads, ffn, t)
    T = B * S
    gemm = {
        "gemm_qkv": 2 * T * hidden * (hl + 2 * kvl) * d,
        "gemm_out": 2 * T * hl * d * hidden,
        "gemm_up": 2 * T * hidden * 2 * fl,
        "gemm_down": 2 * T * fl * hidden,
    }
    attn = 2 * B * hl * S * S * d
    return gemm, attn


def weight_bytes(hidden, heads, kv_heads, ffn, t, fp8=False):
    """Bytes of a rank's four projection weights as decode reads them: bf16,
    or E4M3 codes plus one fp32 scale per row."""
    d, hl, kvl, fl = dims(hidden, heads, kv_heads, ffn, t)
    shapes = [((hl + 2 * kvl) * d, hidden), (hidden, hl * d), (2 * fl, hidden), (hidden, fl)]
    if fp8:
        return sum(n * k + 4 * n for n, k in shapes)
    return sum(2 * n * k for n, k in shapes)


def decode_bytes(hidden, heads, kv_heads, ffn, t, B, L, fp8=False):
    """Algorithmic HBM bytes of one decode step (one token for each of B
    sequences) on one rank at cache length L: the rank's weights once (bf16,
    or E4M3 codes + row scales), K/V of positions 0..L read, one K/V position
    written per sequence (activations are a few KB per sequence and left
    out)."""
    d, hl, kvl, fl = dims(hidden, heads, kv_heads, ffn, t)
    kv_read = B * 2 * 2 * kvl * d * (L + 1)
    wb = (lambda n, k: n * k + 4 * n) if fp8 else (lambda n, k: 2 * n * k)
    per_kernel = {
        "gemv_qkv": wb((hl + 2 * kvl) * d, hidden),
        "gemv_out": wb(hidden, hl * d),
        "gemv_up": wb(2 * fl, hidden),
        "gemv_down": wb(hidden, fl),
        "attn_decode": kv_read,
    }
    return weight_bytes(hidden, heads, kv_heads, ffn, t, fp8) + kv_read + B * 2 * 2 * kvl * d, per_kernel


# ---------------------------------------------------------------- timing

def source_sha(name):
    """Hash of a kernel source together with the headers it includes."""
    h = hashlib.sha256()
    for f in (name, "common.h", "kernels.h", "types.h"):
        h.update(open(os.path.join(ROOT, "tensor_transformer_layer_tp_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(key, src):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(key)
    if not rec or rec.get("source_sha") != source_sha(src):
        return None
    return rec.get("bytes_per_launch")


def timed(torch, fn, steps, warmup, stream):
    """Mean ms per step over `steps` back-to-back steps (one event pair
    around all of them), and the median / p10 / p90 of per-step times from
    events recorded between the steps."""
    import numpy as np
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    total = ev[0].elapsed_time(ev[-1])
    return total / steps, {"median": round(float(np.median(per)), 4), "p10": round(float(np.percentile(per, 10)), 4),
                           "p90": round(float(np.percentile(per, 90)), 4)}


def rounded(d):
    return {k: (round(v, 3) if isinstance(v, float) else v) for k, v in d.items()}


class ClockSampler:
    """The GPU clock while a step runs, from amdsmi's GPU metrics table (per-XCD
    current GFX clocks and socket power), when amdsmi is present.  The
    firmware refreshes that table about once a second, so a sample counts
    only once the table's timestamp has moved past its value at the start;
    the caller keeps the GPU busy for a few seconds."""

    def __init__(self):
        self.ok, self.samples = False, []
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi, self.h = amdsmi, amdsmi.amdsmi_get_processor_handles()[0]
            self.t0 = self.read()["stamp"]
            self.ok = True
        except Exception:
            pass

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        clks = [c for c in m.get("current_gfxclks") or [] if isinstance(c, (int, float))]
        return {"stamp": m.get("system_clock_counter"), "mhz": sum(clks) / len(clks) if clks else None,
                "power": m.get("current_socket_power")}

    def __enter__(self):
        if self.ok:
            import threading
            self.stop = threading.Event()

            def run():
                last = self.t0
                while not self.stop.is_set():
                    try:
                        r = self.read()
                        if r["stamp"] != last and r["mhz"]:
                            last = r["stamp"]
                            self.samples.append(r)
                    except Exception:
                        pass
                    time.sleep(0.01)

            self.thread = threading.Thread(target=run, daemon=True)
            self.thread.start()
        return self

    def __exit__(self, *exc):
        if self.ok:
            self.stop.set()
            self.thread.join()

    def summary(self):
        import numpy as np
        if not self.samples:
            return None
        mhz = np.array([r["mhz"] for r in self.samples])
        pw = [r["power"] for r in self.samples if isinstance(r["power"], (int, float))]
        return {"median_MHz": round(float(np.median(mhz)), 1), "min_MHz": round(float(mhz.min()), 1),
                "max_MHz": round(float(mhz.max()), 1), "socket_power_W": float(np.median(pw)) if pw else None,
                "samples": int(mhz.size),
                "source": "amdsmi GPU metrics (mean of the per-XCD current GFX clocks), fresh refreshes during "
                          "a ~2.5 s run of back-to-back steps"}


def clock_pass(torch, step, seconds=2.5):
    """Runs `step` back to back for about `seconds` while sampling the clock."""
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    return clock.summary()


NOMINAL_CLOCK_MHZ = 2400.0     # the clock the 2.5 PFLOP/s bf16 peak assumes


def copy_ceiling(torch, mib=4096, reps=5):
    """HBM streaming ceiling: the best rate of a plain device copy of `mib` MiB
    (bytes read + bytes written over the copy's event-timed duration)."""
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 1e30
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * n / (best * 1e-3) / 1e9, 1)


# ---------------------------------------------------------------- prefill

def prefill_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, x, exact_others, kv_cap=None, fused=False):
    """Rank 0's shard plus the buffers of one prefill step.  The other
    ranks' partials are either computed by their own shards once
    (exact_others) or seeded N(0, 0.1^2) stand-ins (timing only).  With
    `fused`, each stage's reduce runs in its row-parallel projection's
    epilogue and a norm kernel follows; otherwise the stage stores its
    partial and a reduce kernel with the norm fused follows.  Returns the
    shard, the cache, the step and the other variant's step."""
    from tensor_transformer_layer_tp_amd import ATTN, MLP, PRENORM, Shard, partial_reduce
    B, S = int(x.shape[0]), int(x.shape[1])
    sh = Shard(hidden, heads, kv_heads, ffn, t, 0)
    sh.load_weights(wdev)
    sh.reserve(B * S)
    kv = sh.kv_cache(B, kv_cap or S)
    pa = [torch.empty((B, S, hidden), dtype=torch.float32, device="cuda") for _ in range(t)]
    pm = [torch.empty((B, S, hidden), dtype=torch.float32, device="cuda") for _ in range(t)]
    hbuf = torch.empty_like(x)
    ybuf = torch.empty_like(x)
    n2buf = torch.empty_like(x)
    n1next = torch.empty_like(x)
    if exact_others:
        for r in range(1, t):
            o = Shard(hidden, heads, kv_heads, ffn, t, r)
            o.load_weights(wdev)
            o.prefill(ATTN, x, None, out=pa[r])
            torch.cuda.synchronize()
            o.close()
        sh.prefill(ATTN, x, kv, out=pa[0])
        partial_reduce(pa, residual=x, out=hbuf)
        for r in range(1, t):
            o = Shard(hidden, heads, kv_heads, ffn, t, r)
            o.load_weights(wdev)
            o.prefill(MLP, hbuf, out=pm[r])
            torch.cuda.synchronize()
            o.close()
    else:
        g = torch.Generator(device="cuda")
        g.manual_seed(99)
        for r in range(1, t):
            pa[r].normal_(0.0, 0.1, generator=g)
            pm[r].normal_(0.0, 0.1, generator=g)
    # the layer input's norm, made once: in a stack of layers the previous
    # layer's last reduce produces it (as every step below does for the next)
    n1 = sh.norm(1, x)
    torch.cuda.synchronize()

    def step_reduce_norm():
        # ATTN stage on the normalised input, the reduce with the MLP stage's
        # norm, the MLP stage, the reduce with the next layer's input norm
        sh.prefill(ATTN | PRENORM, n1, kv, out=pa[0])
        sh.reduce_norm(2, pa, residual=x, out=hbuf, norm_out=n2buf)
        sh.prefill(MLP | PRENORM, n2buf, out=pm[0])
        sh.reduce_norm(1, pm, residual=hbuf, out=ybuf, norm_out=n1next)

    oth_a, oth_m = [None] + pa[1:], [None] + pm[1:]

    def step_fused():
        # the same layer with each reduce in the row-parallel projection's
        # epilogue, then the next stage's norm
        sh.prefill_reduce(ATTN | PRENORM, n1, oth_a, residual=x, kv=kv, out=hbuf)
        sh.norm(2, hbuf, out=n2buf)
        sh.prefill_reduce(MLP | PRENORM, n2buf, oth_m, residual=hbuf, out=ybuf)
        sh.norm(1, ybuf, out=n1next)

    if fused:
        return sh, kv, step_fused, step_reduce_norm
    return sh, kv, step_reduce_norm, step_fused


def bench_prefill(args, torch, name, hidden, heads, kv_heads, ffn, t, wdev, x, exact_others, roof_key, fused=False):
    """Times the rank-0 prefill step; the timed pass brackets only the
    dominant kernel (gate/up GEMM) with events, a second pass brackets
    every kernel for the per-kernel breakdown, a third times the step with
    the other placement of the reduces (unbracketed)."""
    B, S = int(x.shape[0]), int(x.shape[1])
    sh, kv, step, other = prefill_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, x, exact_others, fused=fused)
    stream = torch.cuda.current_stream()
    dom = "gemm_up"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sh.timing(True, kinds=[dom])
    ms, dist = timed(torch, step, args.steps, 0, stream)
    dom_times = sh.timing_read()[dom]
    sh.timing(False)
    clk = clock_pass(torch, step)
    sh.timing(True)
    ms_marked, _ = timed(torch, step, args.steps, 0, stream)
    ktimes = sh.timing_read()
    sh.timing(False)
    for _ in range(min(args.warmup, 5)):
        other()
    ms_other, dist_other = timed(torch, other, args.steps, 0, stream)
    kv.close()
    sh.close()
    gemm, attn = prefill_flops(hidden, heads, kv_heads, ffn, t, B, S)
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
    d, hl, kvl, fl = dims(hidden, heads, kv_heads, ffn, t)
    roof_clock = {}
    if clk:
        peak_clk = PEAK_BF16_TFLOPS * clk["median_MHz"] / NOMINAL_CLOCK_MHZ
        roof_clock = {"peak_at_measured_clock": round(peak_clk, 1), "frac_at_measured_clock": round(achieved / peak_clk, 4)}
    return {
        "clock": clk,
        "workload": name,
        "ms_per_step": round(ms, 4),
        "step_ms": dist,
        "tflops": round(total / (ms * 1e-3) / 1e12, 2),
        "mfma_frac": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": total,
        # with the reduces in the epilogues, the out and down projections' times include them
        "gemm_times_include_reduces": fused,
        "gemm_tflops": round(sum(gemm.values()) / (gemm_us * 1e-6) / 1e12, 2),
        "gemm_mfma_frac": round(sum(gemm.values()) / (gemm_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_all_kernels_bracketed": round(ms_marked, 4),
        "reduce_placement": ("in the row-parallel projections' epilogues, then a norm kernel" if fused
                             else "a reduce kernel with the next norm fused, after each stage"),
        ("ms_per_step_reduce_kernel" if fused else "ms_per_step_reduce_in_epilogue"): round(ms_other, 4),
        "kernels": {k: rounded(v) for k, v in kern.items()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(roof_key, "gemm_bf16.hip"),
                     "kernel": f"gemm (gate/up projection + SwiGLU epilogue), M={B * S} N={2 * fl} K={hidden}",
                     "avg_us": round(dom_us, 3), "launches": dom_times[1], "flops_per_launch": gemm[dom],
                     **roof_clock},
    }


def bench_sp(args, torch, hidden, heads, kv_heads, ffn, t, wdev, x):
    """The sequence-parallel step of rank 0: norm of its T/t token rows,
    all-gather of the ranks' normalised rows, ATTN stage without its norm,
    reduce-scatter, the same for the MLP stage.  The other ranks'
    contributions are seeded stand-ins (timing only)."""
    from tensor_transformer_layer_tp_amd import (ATTN, MLP, PRENORM, Shard, all_gather,
                                                 partial_reduce_scatter)
    B, S = int(x.shape[0]), int(x.shape[1])
    T, n = B * S, B * S // t
    sh = Shard(hidden, heads, kv_heads, ffn, t, 0)
    sh.load_weights(wdev)
    sh.reserve(T)
    kv = sh.kv_cache(B, S)
    g = torch.Generator(device="cuda")
    g.manual_seed(97)
    x0 = x.reshape(T, hidden)[:n].contiguous()
    others_n = [torch.randn((n, hidden), device="cuda", generator=g).to(torch.bfloat16) for _ in range(t - 1)]
    pa = [torch.randn((B, S, hidden), device="cuda", generator=g) * 0.1 for _ in range(t)]
    pm = [torch.randn((B, S, hidden), device="cuda", generator=g) * 0.1 for _ in range(t)]
    n1r, n2r = torch.empty_like(x0), torch.empty_like(x0)
    n1 = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
    n2 = torch.empty_like(n1)
    hr, yr = torch.empty_like(x0), torch.empty_like(x0)

    def step():
        sh.norm(1, x0, out=n1r)
        all_gather([n1r, *others_n], out=n1)
        sh.prefill(ATTN | PRENORM, n1.reshape(B, S, hidden), kv, out=pa[0])
        partial_reduce_scatter(pa, 0, x0, out=hr)
        sh.norm(2, hr, out=n2r)
        all_gather([n2r, *others_n], out=n2)
        sh.prefill(MLP | PRENORM, n2.reshape(B, S, hidden), out=pm[0])
        partial_reduce_scatter(pm, 0, hr, out=yr)

    ms, dist = timed(torch, step, args.steps, args.warmup, torch.cuda.current_stream())
    kv.close()
    sh.close()
    gemm, attn = prefill_flops(hidden, heads, kv_heads, ffn, t, B, S)
    return {"workload": "sequence-parallel step of the same 7B t=2 rank-0 shard: norms on its 1024 token rows, "
                        "all-gather, stages without their norms, reduce-scatter",
            "ms_per_step": round(ms, 4), "step_ms": dist,
            "tflops": round((sum(gemm.values()) + attn) / (ms * 1e-3) / 1e12, 2)}


# ---------------------------------------------------------------- decode

def decode_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, B, L0, cap, copies, fill, fp8=False, block=0):
    """`copies` distinct rank-0 shards (their weights rotate through HBM)
    with caches at length L0; fill(kv) writes the first copy's cache
    content, the others copy it.  block > 0: paged caches of that block
    size with a scrambled block table."""
    import numpy as np
    from tensor_transformer_layer_tp_amd import Shard
    layers = []
    for i in range(copies):
        sh = Shard(hidden, heads, kv_heads, ffn, t, 0, decode_fp8=fp8)
        sh.load_weights(wdev)
        if block:
            mb = -(-cap // block)
            kv = sh.kv_cache_paged(B, cap, block, B * mb)
            kv.set_block_table(np.random.default_rng(5).permutation(B * mb).reshape(B, mb))
        else:
            kv = sh.kv_cache(B, cap)
        if i == 0:
            fill(kv)
        else:
            kv.copy_from(layers[0][1])
        kv.length = L0
        layers.append((sh, kv))
    torch.cuda.synchronize()
    return layers


def decode_step_fn(torch, layers, hidden, t, B, x0, fused=True):
    """One decode token for B sequences through every layer copy: ATTN stage,
    reduce, MLP stage, reduce (other ranks' partials are fixed stand-ins).
    fused: each stage's reduce folded into its row-parallel projection
    (tp_shard_forward_decode_reduce); else the stage, then tp_partial_reduce."""
    from tensor_transformer_layer_tp_amd import ATTN, MLP, partial_reduce
    g = torch.Generator(device="cuda")
    g.manual_seed(98)
    others = [torch.randn((B, hidden), device="cuda", dtype=torch.float32, generator=g) * 0.1 for _ in range(t - 1)]
    pa = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    pm = torch.empty_like(pa)
    hb = torch.empty_like(x0)
    yb = [torch.empty_like(x0) for _ in range(2)]
    slots = [None, *others]   # rank 0's own slot

    def step():
        x = x0
        for i, (sh, kv) in enumerate(layers):
            y = yb[i & 1]
            if fused:
                sh.decode_reduce(ATTN, x, slots, residual=x, kv=kv, out=hb)
                sh.decode_reduce(MLP, hb, slots, residual=hb, out=y)
            else:
                sh.decode(ATTN, x, kv, out=pa)
                partial_reduce([pa, *others], residual=x, out=hb)
                sh.decode(MLP, hb, out=pm)
                partial_reduce([pm, *others], residual=hb, out=y)
            x = y

    return step


def capture(torch, fn):
    """fn's launches recorded in a HIP graph (fn must have run once eagerly
    with the same shapes, so that nothing is allocated during capture)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bench_decode(args, torch, name, hidden, heads, kv_heads, ffn, t, wdev, L0, fill, x0, roof_key, fp8=False,
                 block=0):
    """Decode through a stack of layer copies: eager calls, then the same
    step captured once in a HIP graph and replayed (each replay appends one
    token per layer: the kernels read and advance the device-resident cache
    length), then a per-kernel breakdown pass with event markers."""
    wb = weight_bytes(hidden, heads, kv_heads, ffn, t, fp8)
    nl = args.decode_layers or max(2, -(-int(MIN_DECODE_FOOTPRINT) // wb))
    cap = L0 + 4 * (args.warmup + args.steps) + 8
    layers = decode_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, 1, L0, cap, nl, fill, fp8, block)
    stream = torch.cuda.current_stream()
    step = decode_step_fn(torch, layers, hidden, t, 1, x0)
    ms, dist = timed(torch, step, args.steps, args.warmup, stream)
    g = capture(torch, step)
    gms, gdist = timed(torch, g.replay, args.steps, args.warmup, torch.cuda.current_stream())
    del g
    # the same step with each reduce as its own launch, for comparison
    step2 = decode_step_fn(torch, layers, hidden, t, 1, x0, fused=False)
    step2()
    g2 = capture(torch, step2)
    g2ms, _ = timed(torch, g2.replay, args.steps, args.warmup, torch.cuda.current_stream())
    del g2
    for sh, _ in layers:
        sh.timing(True)
    timed(torch, step, args.steps, 0, stream)
    agg = {}
    for sh, _ in layers:
        for k, (tot, n) in sh.timing_read().items():
            a = agg.setdefault(k, [0.0, 0])
            a[0] += tot
            a[1] += n
        sh.timing(False)
    for sh, kv in layers:
        kv.close()
        sh.close()
    L_avg = L0 + 2 * (args.warmup + args.steps)   # mean cache length over the timed passes
    nbytes, per_kernel = decode_bytes(hidden, heads, kv_heads, ffn, t, 1, int(L_avg), fp8)
    us, us_graph = 1e3 * ms / nl, 1e3 * gms / nl
    kern = {k: {"avg_us": 1e3 * v[0] / v[1], "launches": v[1]} for k, v in agg.items()}
    for k, b in per_kernel.items():
        if k in kern:
            kern[k]["GBps"] = b / (kern[k]["avg_us"] * 1e-6) / 1e9
    dom = "gemv_up"
    ach = per_kernel[dom] / (kern[dom]["avg_us"] * 1e-6) / 1e9
    d, hl, kvl, fl = dims(hidden, heads, kv_heads, ffn, t)
    best = min(us, us_graph)
    return {
        "workload": f"{name}{', E4M3 weights (per-row scales)' if fp8 else ''}"
                    f"{f', paged cache ({block}-position blocks, scrambled table)' if block else ''}, "
                    f"{nl} distinct layer copies ({nl * wb / 1e9:.2f} GB of weights)",
        "us_per_token_layer": round(best, 3),
        "us_per_token_layer_eager": round(us, 3),
        "us_per_token_layer_graph": round(us_graph, 3),
        "us_per_token_layer_graph_separate_reduce": round(1e3 * g2ms / nl, 3),
        "step_ms": dist,
        "step_ms_graph": gdist,
        "bytes_per_token_layer": nbytes,
        "hbm_GBps": round(nbytes / (best * 1e-6) / 1e9, 1),
        "hbm_frac": round(nbytes / (best * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "kernels": {k: rounded(v) for k, v in kern.items()},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4),
                     "traffic": None if fp8 else traffic_for(roof_key, "decode.hip"),
                     "kernel": f"gemv_kernel ({'E4M3' if fp8 else 'bf16'} gate/up + SwiGLU, fused RMSNorm), "
                               f"N={2 * fl} K={hidden}",
                     "bytes_per_launch": per_kernel[dom]},
    }


# ---------------------------------------------------------------- workloads

def run_7b(args, torch):
    from tensor_transformer_layer_tp_amd import synth
    w = synth.WORKLOADS["7b-t2-prefill"]
    raw = synth.draw_workload(w)
    dev = {k: synth.to_storage(v, "bf16").cuda() for k, v in raw.items()}
    wdev = {k: v for k, v in dev.items() if k != "x"}
    pre = bench_prefill(args, torch,
                        "7b-t2-prefill: rank 0 of a 7B-shaped layer split t=2 (hidden 4096, 16 of 32 heads x 128, "
                        "SwiGLU 5504 of 11008), bf16, batch 1 x seq 2048, causal; the other rank's partials computed "
                        "by its own shard", w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, dev["x"], True,
                        "gemm_up_7b_t2")
    pre["sequence_parallel"] = bench_sp(args, torch, w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, dev["x"])
    del dev, wdev
    return pre, (w, raw)


def run_7b_decode(args, torch):
    from tensor_transformer_layer_tp_amd import synth
    w = synth.WORKLOADS["7b-t4-decode"]
    raw = synth.draw_workload(w)
    dev = {k: synth.to_storage(v, "bf16").cuda() for k, v in raw.items()}
    wdev = {k: v for k, v in dev.items() if k not in ("k_cache", "v_cache", "x_dec")}
    kvl = w.kv_heads // w.tp

    def fill(kv):
        kf = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
        vf = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
        kf[:, :, :w.kv_len] = dev["k_cache"][:, :kvl]
        vf[:, :, :w.kv_len] = dev["v_cache"][:, :kvl]
        kv.write(kf, vf)

    name = ("7b-t4-decode: hidden 4096, rank 0 of t=4 (8 of 32 heads x 128, SwiGLU 2752 of 11008), bf16, batch 1, "
            f"cache {w.kv_len}+ positions")
    dec = bench_decode(args, torch, name, w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, w.kv_len, fill,
                       dev["x_dec"], "gemv_up_7b_t4")
    dec8 = bench_decode(args, torch, name, w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, w.kv_len, fill,
                        dev["x_dec"], "gemv8_up_7b_t4", fp8=True)

    def fill_pages(kv):   # the pool holds N(0,1) rows (timing only)
        g = torch.Generator(device="cuda")
        g.manual_seed(6)
        kv.write(torch.randn(kv.shape, generator=g, device="cuda").to(torch.bfloat16),
                 torch.randn(kv.shape, generator=g, device="cuda").to(torch.bfloat16))

    decp = bench_decode(args, torch, name, w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, w.kv_len, fill_pages,
                        dev["x_dec"], "gemv_up_7b_t4_paged", block=16)
    return dec, dec8, decp


def run_70b(args, torch):
    """Rank 0 of the 70B-shaped GQA layer at t=8; inputs drawn on the device
    (timing only: their values do not change the work)."""
    from tensor_transformer_layer_tp_amd import synth
    w = synth.WORKLOADS["70b-t8-prefill"]
    wdev = synth.draw_layer_device(w.hidden, w.heads, w.kv_heads, w.ffn, seed=0)
    x = synth.draw_normal_device((w.batch, w.seq, w.hidden), 1)
    pre = bench_prefill(args, torch,
                        "70b-t8-prefill: rank 0 of a 70B-shaped GQA layer split t=8 (hidden 8192, 8 of 64 query "
                        "heads + 1 of 8 KV heads x 128, SwiGLU 3584 of 28672), bf16, batch 4 x seq 4096, causal",
                        w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, wdev, x, False, "gemm_up_70b_t8", fused=True)
    del x
    dec = None
    if not args.no_decode:
        wd = synth.WORKLOADS["70b-t8-decode"]
        kvl = wd.kv_heads // wd.tp
        d = wd.hidden // wd.heads

        def fill(kv):
            kf = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
            vf = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
            kf[:, :, :wd.kv_len] = synth.draw_normal_device((1, kvl, wd.kv_len, d), 2)
            vf[:, :, :wd.kv_len] = synth.draw_normal_device((1, kvl, wd.kv_len, d), 3)
            kv.write(kf, vf)

        x0 = synth.draw_normal_device((1, wd.hidden), 4)
        name = ("70b-t8-decode: rank 0 of t=8 (8 query heads on 1 KV head x 128, SwiGLU 3584 of 28672), "
                f"bf16, batch 1, cache {wd.kv_len}+ positions")
        dec = (bench_decode(args, torch, name, wd.hidden, wd.heads, wd.kv_heads, wd.ffn, wd.tp, wdev, wd.kv_len,
                            fill, x0, "gemv_up_70b_t8"),
               bench_decode(args, torch, name, wd.hidden, wd.heads, wd.kv_heads, wd.ffn, wd.tp, wdev, wd.kv_len,
                            fill, x0, "gemv8_up_70b_t8", fp8=True))
    return pre, dec


# ---------------------------------------------------------------- crossover sweep

def allreduce_model_us(nbytes):
    """Labelled model, not a measurement: one t=2 all-reduce of nbytes over
    one xGMI link (each GPU sends half and receives half twice = nbytes)."""
    return ALLREDUCE_LATENCY_US + nbytes / (XGMI_LINK_GBPS * 1e9) * 1e6


def kernel_avgs(shards):
    """{kernel kind: mean µs per launch} over the shards' event timers (then
    switched off)."""
    agg = {}
    for sh in shards:
        for k, (tot, n) in sh.timing_read().items():
            a = agg.setdefault(k, [0.0, 0])
            a[0] += tot
            a[1] += n
        sh.timing(False)
    return {k: round(1e3 * v[0] / v[1], 2) for k, v in agg.items()}


def sweep_point(args, torch, wdev, hidden, heads, kv_heads, ffn, t, B, S):
    """Prefill of B x S tokens and decode of one token per sequence at cache
    length S: mean, median and p10/p90 over the timed steps, then one more
    pass with every kernel bracketed by events for the per-kernel means."""
    from tensor_transformer_layer_tp_amd import synth
    stream = torch.cuda.current_stream()
    x = synth.draw_normal_device((B, S, hidden), 1000 + B * 10000 + S)
    extra = 16                                   # decode steps the caches leave room for
    sh, kv, step, _ = prefill_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, x, False, kv_cap=S + extra)
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    est = time.perf_counter() - t0
    n = max(3, min(args.steps, int(0.5 / max(est, 1e-6))))
    ms, dist = timed(torch, step, n, 1, stream)
    sh.timing(True)
    timed(torch, step, n, 0, stream)
    pre_k = kernel_avgs([sh])
    gemm, attn = prefill_flops(hidden, heads, kv_heads, ffn, t, B, S)
    pre = {"ms": ms, "dist": dist, "kernels_us": pre_k,
           "tflops": (sum(gemm.values()) + attn) / (ms * 1e-3) / 1e12}
    del step
    # decode one token per sequence from cache length S over the cache this
    # prefill left, through enough layer copies to span >= 1 GB of weights
    wb = weight_bytes(hidden, heads, kv_heads, ffn, t)
    nl = max(2, -(-int(MIN_DECODE_FOOTPRINT) // wb))
    layers = decode_stack(torch, hidden, heads, kv_heads, ffn, t, wdev, B, S, S + extra, nl,
                          lambda k: k.copy_from(kv))
    kv.close()
    sh.close()
    del x
    x0 = synth.draw_normal_device((B, hidden), 7)
    dstep = decode_step_fn(torch, layers, hidden, t, B, x0)
    nd = max(3, min(args.steps, 6))
    dms, ddist = timed(torch, dstep, nd, 2, stream)
    for s_, _ in layers:
        s_.timing(True)
    timed(torch, dstep, 1, 0, stream)
    dec_k = kernel_avgs([s_ for s_, _ in layers])
    us = 1e3 * dms / nl
    nbytes, _ = decode_bytes(hidden, heads, kv_heads, ffn, t, B, S + 2 + nd // 2)
    dec = {"us": us, "dist_us": {k: round(1e3 * v / nl, 2) for k, v in ddist.items()}, "kernels_us": dec_k,
           "GBps": nbytes / (us * 1e-6) / 1e9}
    for s_, k_ in layers:
        k_.close()
        s_.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return pre, dec


def run_sweep(args, torch):
    """7B-shaped layer: rank 0 of t=2 against the unsharded layer (t=1) on
    the same GPU and kernels, prefill of B x S tokens and decode of one
    token per sequence at cache length S, timed separately."""
    from tensor_transformer_layer_tp_amd import synth
    hidden, heads, kv_heads, ffn = 4096, 32, 32, 11008
    wdev = synth.draw_layer_device(hidden, heads, kv_heads, ffn, seed=0)
    res = {}
    for t in (2, 1):
        for B in synth.SWEEP_BATCH:
            for S in synth.SWEEP_SEQ:
                print(f"[sweep] t={t} B={B} S={S}", file=sys.stderr, flush=True)
                res[(t, B, S)] = sweep_point(args, torch, wdev, hidden, heads, kv_heads, ffn, t, B, S)
    table = []
    for B in synth.SWEEP_BATCH:
        for S in synth.SWEEP_SEQ:
            p2, d2 = res[(2, B, S)]
            p1, d1 = res[(1, B, S)]
            msg_pre = B * S * hidden * 2          # bf16 [T, h] per all-reduce
            msg_dec = B * hidden * 2
            table.append({
                "B": B, "S": S,
                "prefill_ms_t2": round(p2["ms"], 4), "prefill_ms_t1": round(p1["ms"], 4),
                "prefill_step_ms_t2": p2["dist"], "prefill_step_ms_t1": p1["dist"],
                "prefill_kernels_us_t2": p2["kernels_us"], "prefill_kernels_us_t1": p1["kernels_us"],
                "prefill_ratio": round(p2["ms"] / p1["ms"], 3),
                "prefill_tflops_t2": round(p2["tflops"], 1), "prefill_tflops_t1": round(p1["tflops"], 1),
                "decode_us_t2": round(d2["us"], 2), "decode_us_t1": round(d1["us"], 2),
                "decode_step_us_t2": d2["dist_us"], "decode_step_us_t1": d1["dist_us"],
                "decode_kernels_us_t2": d2["kernels_us"], "decode_kernels_us_t1": d1["kernels_us"],
                "decode_ratio": round(d2["us"] / d1["us"], 3),
                "decode_GBps_t2": round(d2["GBps"], 1), "decode_GBps_t1": round(d1["GBps"], 1),
                "model_allreduce_us_prefill_t2": round(2 * allreduce_model_us(msg_pre), 1),
                "model_allreduce_us_decode_t2": round(2 * allreduce_model_us(msg_dec), 1),
            })
    return table


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(state):
    """The CPU oracle (NumPy float64) on the same rank-0 prefill step; the
    other rank's partials are computed first, outside the timed part."""
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
    while steps < 30 and (t_tot < 10.0 or steps == 0):
        t0 = time.perf_counter()
        a0 = O.attn_stage(x, ex, spec, w.tp, 0)["partial"]
        hh = O.reduce([a0, a1], x, spec)
        m0 = O.mlp_stage(hh, ex, spec, w.tp, 0)["partial"]
        O.reduce([m0, m1], hh, spec)
        t_tot += time.perf_counter() - t0
        steps += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return steps, t_tot, threads


def cpu_baseline_70b():
    """The CPU oracle (NumPy float64) on a bounded sample of the headline
    workload: one of the four sequences (S = 4096) of the 70B t=8 rank-0
    step, whole -- ATTN stage, reduce over eight partials, MLP stage,
    reduce -- repeated until 10 s.  The seven other ranks' partials are
    seeded stand-ins made before timing (the reduce's arithmetic is the
    same).  Only rank 0's blocks of the full weight matrices are drawn and
    read; the oracle slices them out of full-shape arrays itself."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import layer as O
    from tensor_transformer_layer_tp_amd import synth
    w = synth.WORKLOADS["70b-t8-prefill"]
    spec = O.Spec(w.hidden, w.heads, w.kv_heads, w.ffn)
    d, hl, kvl, fl = dims(w.hidden, w.heads, w.kv_heads, w.ffn, w.tp)
    h = w.hidden
    rng = np.random.default_rng(0)

    def draw(shape, scale):
        return O.bf16_round(rng.standard_normal(shape) * scale)

    W = {k: np.empty(shp) for k, shp in (("wq", (w.heads * d, h)), ("wk", (w.kv_heads * d, h)),
                                         ("wv", (w.kv_heads * d, h)), ("wo", (h, w.heads * d)),
                                         ("w_gate", (w.ffn, h)), ("w_up", (w.ffn, h)), ("w_down", (h, w.ffn)))}
    W["wq"][:hl * d] = draw((hl * d, h), 0.02)
    W["wk"][:kvl * d] = draw((kvl * d, h), 0.02)
    W["wv"][:kvl * d] = draw((kvl * d, h), 0.02)
    W["wo"][:, :hl * d] = draw((h, hl * d), 0.02)
    W["w_gate"][:fl] = draw((fl, h), 0.02)
    W["w_up"][:fl] = draw((fl, h), 0.02)
    W["w_down"][:, :fl] = draw((h, fl), 0.02)
    W["g1"] = np.ones(h)
    W["g2"] = np.ones(h)
    x = draw((1, w.seq, h), 1.0)
    other = rng.standard_normal((1, w.seq, h)) * 0.1      # stand-in partial of each other rank
    steps, t_tot = 0, 0.0
    while steps < 5 and (t_tot < 10.0 or steps == 0):
        t0 = time.perf_counter()
        a0 = O.attn_stage(x, W, spec, w.tp, 0)["partial"]
        hh = O.reduce([a0] + [other] * (w.tp - 1), x, spec)
        m0 = O.mlp_stage(hh, W, spec, w.tp, 0)["partial"]
        O.reduce([m0] + [other] * (w.tp - 1), hh, spec)
        t_tot += time.perf_counter() - t0
        steps += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    gemm, attn = prefill_flops(w.hidden, w.heads, w.kv_heads, w.ffn, w.tp, 1, w.seq)
    flops = sum(gemm.values()) + attn
    return {
        "value": round(flops * steps / t_tot / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{steps} run(s) of one of the four sequences (1 x 4096 tokens, {flops / 1e9:.0f} GFLOP each) of "
                  f"the 70B t=8 rank-0 prefill step (ATTN stage, reduce over 8 partials, MLP stage, reduce) in "
                  f"NumPy float64, {t_tot:.1f} s on {cpu_model()}",
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---------------------------------------------------------------- profile summaries

# The roofline kernels the profile summaries cover: key -> (source file,
# kernel kind, shape, where the bench line reports it, dispatches of that
# kernel made before the warmup steps, algorithmic bytes per launch).  A
# projection GEMM's kernel name follows from its launch plan; the gate/up
# projection is the only one with the SwiGLU epilogue (template MODE 2).
ROOF_KERNELS = {
    "gemm_up_70b_t8": ("gemm_bf16.hip", "gemm", (16384, 7168, 8192), ("roofline",), 0,
                       2 * (16384 * 8192 + 7168 * 8192 + 16384 * 3584)),
    "gemm_up_7b_t2": ("gemm_bf16.hip", "gemm", (2048, 11008, 4096), ("prefill_7b", "roofline"), 1,
                      2 * (2048 * 4096 + 11008 * 4096 + 2048 * 5504)),
    # traffic only (no bench-line figure): the 70B out and down projections with the reduce of the
    # other seven ranks' partials in the epilogue share one kernel; their algorithmic bytes averaged
    "gemm_sum_70b_t8": ("gemm_bf16.hip", "gemm_sum", (16384, 8192, 0), ("no line figure",), 0,
                        (2 * (16384 * 1024 + 8192 * 1024) + 2 * (16384 * 3584 + 8192 * 3584)) // 2
                        + 16384 * 8192 * (4 * 7 + 2 + 2)),
    "gemv_up_7b_t4": ("decode.hip", "gemv", (5504, 4096), ("decode", "roofline"), 0,
                      2 * (5504 * 4096 + 4096 + 2752)),
    "gemv_up_70b_t8": ("decode.hip", "gemv", (7168, 8192), ("decode_70b", "roofline"), 0,
                       2 * (7168 * 8192 + 8192 + 3584)),
}
# tile configuration -> the kernel template it launches (the planner's choices)
CFG_KERNEL = {11: "gemm_vgpr_kernel<256, 256, 2, 4, ", 12: "gemm_vgpr_kernel<256, 128, 4, 2, ",
              13: "gemm_vgpr_kernel<256, 192, 8, 1, ", 14: "gemm_ws_kernel<256, 256, 2, 4, ",
              15: "gemm_ws_kernel<256, 192, 8, 1, ", 16: "gemm_ws_kernel<256, 128, 4, 2, ",
              17: "gemm_ws_kernel<256, 192, 4, 1, ", 18: "gemm_ws_kernel<256, 128, 4, 1, "}


def roof_patterns(key):
    """Regexes of the launch kinds of one roofline kernel."""
    import re
    _, kind, shape, _, _, _ = ROOF_KERNELS[key]
    if kind == "gemm_sum":
        return [re.escape("gemm_ws_kernel<256, 256, 2, 4, 5>")]
    if kind == "gemv":
        # batch-1 bf16 GEMV with the SwiGLU epilogue and the fused norm; its
        # NI (16-byte chunks per thread) follows from K
        kc = shape[1] // 8
        ni = 1 if kc <= 256 else (kc + 255) // 256
        return [r"gemv_kernel<1, \d+, " + str(ni) + r", 2, true, false, \d+>"]
    from tensor_transformer_layer_tp_amd import gemm_plan
    return [re.escape(CFG_KERNEL[c] + "2>") if c in CFG_KERNEL else r"gemm_\w+_kernel<[^>]*, 2>"
            for c, _ in gemm_plan(*shape, "swiglu")]


def summarize(trace_dir, fetch_dir, write_dir, bench_json, calib_mib):
    """Per-launch HBM bytes of the roofline kernels from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
    the same counter's reading for the known-size copy (--calib-copy), and
    a kernel-duration table from the --kernel-trace --stats run of the same
    bench command, next to the live event timings of its JSON line."""
    import csv
    import glob
    import re
    import statistics

    def rows(d, suffix):
        out = []
        for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
            out.extend(csv.DictReader(open(f)))
        return out

    def dig(obj, path):
        for k in path:
            obj = obj.get(k) if isinstance(obj, dict) else None
        return obj

    calib = calib_mib * 1024 * 1024
    traffic, facts = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rs = sorted((r for r in rows(d, "counter_collection.csv") if r["Counter_Name"] == counter),
                    key=lambda r: int(r["Dispatch_Id"]))
        # the calibration copies are the run's first three large copies (--calib-copy
        # makes them before anything else; the copy-ceiling copies come later)
        copies = [float(r["Counter_Value"]) * 1024 for r in rs
                  if "copy" in r["Kernel_Name"].lower() and float(r["Counter_Value"]) * 1024 > calib / 8][:3]
        if len(copies) < 3:
            raise SystemExit(f"no calibration copies found in {d}")
        factor = calib / statistics.median(copies)
        facts[counter] = factor
        for key in ROOF_KERNELS:
            # one projection may run as several launches (a column split): bytes per
            # projection = all matching dispatches / dispatches of one launch kind
            names = {}
            for r in rs:
                if any(re.search(p, r["Kernel_Name"]) for p in roof_patterns(key)):
                    names.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024 * factor)
            if names:
                calls = max(len(v) for v in names.values())
                traffic.setdefault(key, {})[counter] = (sum(sum(v) for v in names.values()) / calls, calls)
    rec = {}
    for key, (src, _, _, _, _, alg) in ROOF_KERNELS.items():
        if key not in traffic or len(traffic[key]) != 2:
            continue
        f, nf = traffic[key]["FETCH_SIZE"]
        w, nw = traffic[key]["WRITE_SIZE"]
        rec[key] = {"source": src, "source_sha": source_sha(src), "bytes_per_launch": round(f + w),
                    "fetch_bytes": round(f), "write_bytes": round(w), "algorithmic_bytes": alg,
                    "traffic_over_algorithmic": round((f + w) / alg, 3), "launches": [nf, nw],
                    "fetch_factor": round(facts["FETCH_SIZE"], 4), "write_factor": round(facts["WRITE_SIZE"], 4)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    # kernel durations from the trace run, next to the bench's live event timings
    stats = rows(trace_dir, "kernel_stats.csv")
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    disp = sorted(rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
    md = ["| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in stats[:30]:
        name = r["Name"].replace("|", "/")
        name = name if len(name) <= 110 else name[:107] + "..."
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    live = []
    lo_w, k = int(line["warmup"]), int(line["steps"])
    for key, (_, kind, _, path, skip, _) in ROOF_KERNELS.items():
        roof = dig(line, path)
        if not roof:
            continue
        pats = roof_patterns(key)
        kinds = [r for r in stats if any(re.search(p, r["Name"]) for p in pats)]
        if not kinds:
            continue
        if kind == "gemm":
            # the timed window: `skip` earlier launches, `warmup` untimed steps,
            # then the `steps` timed ones (one projection per step)
            window = 0.0
            for r in kinds:
                d = [int(x["End_Timestamp"]) - int(x["Start_Timestamp"]) for x in disp if x["Kernel_Name"] == r["Name"]]
                lo = skip + lo_w
                window += statistics.mean(d[lo:lo + k]) / 1e3 if len(d) >= lo + k else float("nan")
            allavg = sum(float(r["AverageNs"]) for r in kinds) / 1e3
            names = ", ".join(re.search(r"gemm_\w+_kernel<[^>]*>", r["Name"]).group(0) for r in kinds)
            live.append(f"- `{key}` ({roof['kernel']}): live HIP-event average {roof['avg_us']} µs over the "
                        f"{roof['launches']} timed projections; rocprof over the same {k} dispatches (after "
                        f"{skip} earlier launch(es) and the {lo_w} warmup steps): {window:.1f} µs; over all "
                        f"{kinds[0]['Calls']} dispatches of the run: {allavg:.1f} µs "
                        f"({names})")
        else:
            dk = dig(line, path[:-1] + ("kernels",)) or {}
            gv = dk.get("gemv_up", {})
            live.append(f"- `{key}` ({roof['kernel']}): live HIP-event average {gv.get('avg_us')} µs over "
                        f"{gv.get('launches')} launches; rocprof {float(kinds[0]['AverageNs']) / 1e3:.1f} µs (events "
                        f"bracketing every short kernel under the tracer inflate the live figure)")
    with open(os.path.join(ROOT, "profiles", "bench_kernel_stats.md"), "w") as fh:
        fh.write("# Kernel durations of `bench.py` (rocprofv3 --kernel-trace --stats)\n\n")
        fh.write("Command: profiles/README.md, command 1.  Bench line of the same run: "
                 f"{line['config']['workload'][:60]}... {line['value']} TFLOP/s, {line['ms_per_step']} ms per "
                 f"step ({line['steps']} steps after {line['warmup']} warmup steps).\n\n")
        fh.write("\n".join(live) + "\n\n" + "\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))


def summarize_mfma(pmc_dir, out_name):
    """MFMA evidence for the prefill kernels from one rocprofv3 --pmc MfmaUtil
    MfmaFlopsBF16 GRBM_GUI_ACTIVE run: per kernel kind the dispatch count,
    mean duration, rocprofv3's MfmaUtil (MFMA busy cycles / (active cycles x
    SIMDs)), the executed bf16 MFMA FLOPs per dispatch and the clock the
    kernel ran at (active cycles per XCD over the duration)."""
    import csv
    import glob
    import re
    import statistics
    rows = []
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    agents = []
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*agent_info.csv"), recursive=True)):
        agents.extend(a for a in csv.DictReader(open(f)) if a.get("Name", "").startswith("gfx"))
    n_xcc = int(agents[0]["Num_Xcc"]) if agents else 8
    disp = {}
    for r in rows:
        name = r["Kernel_Name"]
        if not re.search(r"gemm_\w+_kernel|attn_prefill_(kernel|pipe)", name):
            continue
        d = disp.setdefault((name, r["Dispatch_Id"]),
                            {"name": name, "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    kinds = {}
    for d in disp.values():
        kinds.setdefault(d["name"], []).append(d)
    mode_of = {"0": "fp32 partial (out and down projections)", "1": "Q/K/V + rotary", "2": "gate/up + SwiGLU",
               "5": "out and down + reduce of the partials"}
    md = ["| kernel | dispatches | mean µs | MfmaUtil % | executed bf16 MFMA GFLOP per dispatch | clock GHz |",
          "|---|---:|---:|---:|---:|---:|"]
    for name, ds in sorted(kinds.items(), key=lambda kv: -statistics.mean(x["us"] for x in kv[1])):
        us = statistics.mean(x["us"] for x in ds)
        util = statistics.mean(x.get("MfmaUtil", float("nan")) for x in ds)
        gf = statistics.mean(x.get("MfmaFlopsBF16", float("nan")) for x in ds) / 1e9
        ghz = statistics.mean(x.get("GRBM_GUI_ACTIVE", float("nan")) / n_xcc / (x["us"] * 1e3) for x in ds)
        m = re.search(r"gemm_\w+_kernel<(?:[^>]*, )?(\d)>", name)
        label = (re.search(r"(gemm_\w+_kernel<[^>]*>|attn_prefill_\w*)", name) or re.search(r".*", name)).group(0)
        a = re.search(r"attn_prefill_(kernel|pipe)ILi(\d+)ELi(\d+)E", name)
        if a:
            label = f"attn_prefill_{a.group(1)}<{a.group(2)}, {a.group(3)}> (causal GQA attention)"
        if m:
            label += f" ({mode_of.get(m.group(1), '')})"
        md.append(f"| `{label[:90]}` | {len(ds)} | {us:.1f} | {util:.1f} | {gf:.2f} | {ghz:.2f} |")
    notes = []
    for key, (_, kind, shape, _, _, _) in ROOF_KERNELS.items():
        if kind != "gemm":
            continue
        ex = sum(statistics.mean(x.get("MfmaFlopsBF16", 0.0) for x in kinds[n]) for n in kinds
                 if any(re.search(p, n) for p in roof_patterns(key))) / 1e9
        if ex:
            M, N, K = shape
            notes.append(f"- `{key}` (M={M} N={N} K={K}): {ex:.2f} GFLOP executed by its launch kinds per projection "
                         f"against {2 * M * N * K / 1e9:.2f} algorithmic (zero padding of ragged tiles is the difference)")
    lines = ["# MFMA counters of the prefill kernels (rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 GRBM_GUI_ACTIVE)", "",
             "Command: profiles/README.md. MfmaUtil is rocprofv3's derived counter: MFMA busy cycles over active "
             "cycles times SIMDs, at the clock the kernel ran at; executed FLOPs are SQ_INSTS_VALU_MFMA_MOPS_BF16 x "
             "512; the clock is GRBM_GUI_ACTIVE per XCD over the dispatch duration.", "", *notes, "", *md]
    with open(os.path.join(ROOT, "profiles", out_name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_warmup(pmc_dir, key, out_name):
    """The first dispatches of one roofline GEMM in a fresh process, from a
    rocprofv3 --pmc GRBM_GUI_ACTIVE run: duration and clock (active cycles
    per XCD over the duration) per dispatch, in launch order."""
    import csv
    import glob
    import re
    import statistics
    rows = []
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    pats = roof_patterns(key)
    ds = sorted(({"id": int(r["Dispatch_Id"]), "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
                  "cyc": float(r["Counter_Value"])} for r in rows
                 if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and any(re.search(p, r["Kernel_Name"]) for p in pats)),
                key=lambda d: d["id"])
    _, _, shape, _, _, _ = ROOF_KERNELS[key]
    flops = 2.0 * shape[0] * shape[1] * shape[2]
    md = ["| dispatch | µs | clock GHz | TFLOP/s |", "|---:|---:|---:|---:|"]
    for i, d in enumerate(ds[:40]):
        md.append(f"| {i} | {d['us']:.1f} | {d['cyc'] / 8 / (d['us'] * 1e3):.3f} | {flops / (d['us'] * 1e-6) / 1e12:.0f} |")
    tail = ds[10:40]
    lines = [f"# First dispatches of `{key}` in a fresh process (rocprofv3 --pmc GRBM_GUI_ACTIVE)", "",
             "Command: profiles/README.md.  Clock = GRBM_GUI_ACTIVE / 8 XCDs / duration.", ""]
    if tail:
        lines.append(f"- dispatches 10-39: mean {statistics.mean(d['us'] for d in tail):.1f} µs; dispatch 0: "
                     f"{ds[0]['us']:.1f} µs, dispatches 1-4: {statistics.mean(d['us'] for d in ds[1:5]):.1f} µs")
    lines += ["", *md]
    with open(os.path.join(ROOT, "profiles", out_name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def synth_workload(name):
    from tensor_transformer_layer_tp_amd import synth
    return synth.WORKLOADS[name]


def calib_copy(torch, mib):
    """A plain device copy of known size (the scale for byte counters)."""
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize, args.calib_copy or 1024)
        return
    if args.summarize_warmup:
        summarize_warmup(*args.summarize_warmup)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs one rank's shard per "
              "device, and the ranks' collectives are not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.calib_copy:
        calib_copy(torch, args.calib_copy)
    if args.sweep:
        table = run_sweep(args, torch)
        print(json.dumps({"sweep": "7B-shaped layer, rank 0 of t=2 vs t=1 (unsharded), bf16; prefill B x S tokens "
                                   "(step = ATTN + reduce + MLP + reduce); decode one token per sequence at cache "
                                   "length S, per layer; model_allreduce_* is a labelled link-bound model of the two "
                                   "all-reduces a real t=2 layer adds, not a measurement",
                          "points": table}), flush=True)
        return
    big = None if args.no_70b else run_70b(args, torch)
    small = None if args.no_7b else run_7b(args, torch)
    dec = None if (args.no_decode or args.no_7b) else run_7b_decode(args, torch)
    if big is None and small is None:
        print("nothing to run (--no-7b and --no-70b)", file=sys.stderr)
        sys.exit(2)
    if big is not None:
        head = big[0]
        config = {
            "workload": "70b-t8-prefill: rank 0 of a 70B-shaped GQA layer split t=8 (hidden 8192, 8 of 64 query heads "
                        "+ 1 of 8 KV heads x 128, SwiGLU 3584 of 28672, RMSNorm, RoPE), bf16, batch 4 x seq 4096, "
                        "causal; step = ATTN stage ending in the reduce of 8 partials (in the out projection's "
                        "epilogue) + the MLP norm + MLP stage ending in the reduce of 8 partials (in the down "
                        "projection's epilogue) + the next layer's input norm",
            "global_batch": 4, "seq_len": 4096, "parallelism": "tp8 shard (rank 0) on 1 GPU",
        }
    else:
        head = small[0]
        w = small[1][0]
        config = {
            "workload": "7b-t2-prefill: rank 0 of a 7B-shaped layer split t=2 (hidden 4096, 16 of 32 heads x 128, "
                        "SwiGLU 5504 of 11008, RMSNorm, RoPE), bf16, batch 1 x seq 2048, causal; step = ATTN stage "
                        "+ reduce with the MLP norm + MLP stage + reduce with the next layer's input norm",
            "global_batch": w.batch, "seq_len": w.seq, "parallelism": "tp2 shard (rank 0) on 1 GPU",
        }
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random-init)",
        "config": config,
    }
    for k in ("step_ms", "mfma_frac", "flops_per_step", "gemm_times_include_reduces", "gemm_tflops",
              "gemm_mfma_frac", "ms_per_step_all_kernels_bracketed", "reduce_placement", "ms_per_step_reduce_kernel",
              "ms_per_step_reduce_in_epilogue", "kernels", "clock", "roofline"):
        if k in head:
            line[k] = head[k]
    line["hbm_copy_GBps"] = copy_ceiling(torch)
    if big is not None and small is not None:
        line["prefill_7b"] = small[0]
    if big is not None and big[1] is not None:
        line["decode_70b"], line["decode_70b_fp8"] = big[1]
    if dec is not None:
        line["decode"], line["decode_fp8"], line["decode_paged"] = dec
    if not args.no_cpu:
        if big is not None:
            line["cpu_baseline"] = cpu_baseline_70b()
        else:
            steps, secs, threads = cpu_baseline(small[1])
            line["cpu_baseline"] = {
                "value": round(head["flops_per_step"] * steps / secs / 1e12, 5), "unit": "TFLOP/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{steps} full rank-0 prefill step(s) of the same workload (B=1, S=2048) in NumPy "
                          f"float64, {secs:.1f} s on {cpu_model()}",
            }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
