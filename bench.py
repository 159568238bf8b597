"""Benchmark: gated SA+SWA forward on one MI355X, long-context layer n = 32768, w = 128.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-cpu-baseline]
    python bench.py --nsweep      (SA against full causal attention, n = 2K .. 32K)
    python bench.py --train       (gated layer training step: forward with lse + backward)
    python bench.py --decode      (gated decode step over a KV cache, batch 128, n_max 32768)
    python bench.py --configs     (every synthetic workload: time per layer, tokens/s, TFLOP/s,
                                   fraction of the HBM roofline)
    python bench.py --gates       (gate projections sigmoid(x w + b), n 32768, Hm 4096, 32 heads)

One step is one pass of the whole hot path over one layer's synthetic input: one call of
ssw_gated_sa_swa_forward, i.e. the SA pass (sigma-gathered window attention, leaves g_sa * Y_sa as
the intermediate at the scattered rows) followed by the SWA pass (adds g_swa * Y_swa).
Workload: B 1, n 32768, 32 query / 8 KV heads, d 128, bf16, causal, w 128; Q, K, V ~ N(0,1),
gates sigmoid(N(0,1)), sigma from the seeded generator.  Inputs are resident in HBM before the
timed region; three copies of every buffer are rotated so that no step finds its operands in
the 256 MB last-level cache from the previous step.  The timed region is K back-to-back steps
bracketed by HIP events on the stream the kernels run on; every fourth of them goes through the
timed form of the entry point, whose events are attached to the two kernels' dispatches, so the
step time and each kernel's average duration (for the roofline) come from the same loop.

Prints ONE JSON line on stdout (details on stderr).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated SA+SWA fwd tokens/s + TFLOP/s, % roofline at n=32K, w=128 (1 GPU)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(n: int, w: int) -> int:
    """Exact number of (query, key) pairs per (batch row, head) of causal SA (and of causal SWA):
    every in-band pair of distinct slots is kept in exactly one direction, plus the n self pairs."""
    w = min(w, n)
    return n * w - w * (w - 1) // 2


def pass_bytes(B, n, Hq, Hkv, d, elem, sa: bool, accumulate: bool) -> int:
    """Algorithmic HBM bytes of one pass: each operand read once, the output written once."""
    q = B * n * Hq * d * elem
    kv = 2 * B * n * Hkv * d * elem
    gate = B * n * Hq * 4
    out = B * n * Hq * d * elem
    sigma = n * 4 if sa else 0
    return q + kv + gate + sigma + out * (2 if accumulate else 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # untimed steps before the timed region: the shader clock moves over the first few dozen
    # steps of a fresh process (measured on one box: 518 us per step over 20 steps after 5
    # warm-up steps, 436 us over 100 steps after 50), so the default reaches the steady state
    # first (about 25 ms)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--window", type=int, default=128)
    ap.add_argument("--sweep", action="store_true", help="also time SA / SWA alone at w 16 .. 512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample size (0 = auto)")
    ap.add_argument("--nsweep", action="store_true",
                    help="instead: SA (w = --window) against full causal attention for n = 2K..32K")
    ap.add_argument("--train", action="store_true",
                    help="instead: the gated layer's training step (forward with lse + backward)")
    ap.add_argument("--decode", action="store_true",
                    help="instead: one gated decode step per batch row over a KV cache")
    ap.add_argument("--batch", type=int, default=128, help="decode batch rows")
    ap.add_argument("--configs", action="store_true",
                    help="instead: every synthetic workload's paths, one JSON line")
    ap.add_argument("--gates", action="store_true",
                    help="instead: the gate projections of the long-context layer")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); the multi-GPU path is "
              "not built -- per-GPU shards are independent (see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    if args.nsweep:
        return nsweep(args)
    if args.train:
        return train(args)
    if args.decode:
        return decode(args)
    if args.configs:
        return all_configs(args)
    if args.gates:
        return gates_bench(args)

    wl = synth.workload(4)
    B, n, Hq, Hkv, d = wl.B, wl.n, wl.Hq, wl.Hkv, wl.d
    w = args.window
    causal = True

    # ---- inputs (host draw, then resident on the device)
    t0 = time.perf_counter()
    q, k, v = synth.qkv(synth.data_seed(4, 0), B, n, Hq, Hkv, d, wl.dtype)
    g = synth.gates(synth.data_seed(4, 0), B, n, Hq)
    log(f"inputs drawn in {time.perf_counter() - t0:.1f}s")
    t0 = time.perf_counter()
    sigma = ssw.make_permutation(synth.sigma_seed(4, 0), n)
    sigma_ms = (time.perf_counter() - t0) * 1e3
    # the oracle's worker processes are forked now, before this process touches the GPU
    pool = None if args.no_cpu_baseline else OraclePool(q, k, v, g, sigma, w, causal)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ROT = 3
    sets = []
    for _ in range(ROT):
        sets.append(dict(q=q.to(dev), k=k.to(dev), v=v.to(dev), gates=g.to(dev),
                         out=torch.empty(B, n, Hq, d, dtype=q.dtype, device=dev),
                         sigma=torch.from_numpy(sigma).to(dev)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(s, ev):
        ssw.gated_sa_swa_forward(s["q"], s["k"], s["v"], s["sigma"], w, causal, s["gates"],
                                 out=s["out"], events=ev)

    # Every fourth timed step goes through the timed form of the entry point: its four events are
    # attached to the two kernels' dispatches (no separate event packets), so the step time and
    # each kernel's duration come from the same timed loop.  Attaching the events costs about
    # 10 us per step (measured: 428 us per step plain, 438 us with events on every step), so they
    # ride on a quarter of the steps; the others are plain calls of the same entry point.
    K = args.steps
    EV_EVERY = 4
    ev_steps = list(range(0, K, EV_EVERY))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in ev_steps}
    for quad in evs.values():  # materialise the (lazily created) HIP events before timing
        for e in quad:
            e.record(stream)
    for i in range(args.warmup):
        step(sets[i % ROT], None)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # ---- the timed region: K steps, back to back
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(sets[i % ROT], evs.get(i))
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    quads = [evs[i] for i in ev_steps]
    swa_each = [e[0].elapsed_time(e[1]) for e in quads]
    sa_each = [e[2].elapsed_time(e[3]) for e in quads]
    swa_ms = float(np.mean(swa_each))
    sa_ms = float(np.mean(sa_each))
    # the step's span (first kernel's start to second kernel's end) over the first and the last
    # quarter of the sampled steps: the shader clock moves over the first few dozen steps of a
    # fresh process, so these show how far the timed region sits from the steady state
    spans = [e[2].elapsed_time(e[1]) for e in quads]
    qn = max(1, len(spans) // 4)
    span_first, span_last = float(np.mean(spans[:qn])), float(np.mean(spans[-qn:]))

    copy_gbs = copy_bandwidth(dev, stream, start, end)

    tokens = B * n
    flops_pass = 4 * d * B * Hq * causal_pairs(n, w)
    # the SA pass runs first and writes the intermediate; the SWA pass reads it and adds
    sa_bytes = pass_bytes(B, n, Hq, Hkv, d, 2, sa=True, accumulate=False)
    swa_bytes = pass_bytes(B, n, Hq, Hkv, d, 2, sa=False, accumulate=True)
    step_bytes = swa_bytes + sa_bytes
    value = tokens / (ms_per_step * 1e-3)
    tflops = 2 * flops_pass / (ms_per_step * 1e-3) / 1e12

    dom = ("sa_pass", sa_ms, sa_bytes) if sa_ms >= swa_ms else ("swa_pass", swa_ms, swa_bytes)
    achieved = dom[2] / (dom[1] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom[0]),
                "kernel": dom[0], "bytes_per_launch": dom[2], "avg_launch_ms": round(dom[1], 4)}
    log(f"step {ms_per_step * 1e3:.1f} us (first quarter of the steps {span_first * 1e3:.1f} us, "
        f"last quarter {span_last * 1e3:.1f} us); "
        f"SWA pass {swa_ms * 1e3:.1f} us = {swa_bytes / swa_ms / 1e6:.0f} GB/s, "
        f"SA pass {sa_ms * 1e3:.1f} us = {sa_bytes / sa_ms / 1e6:.0f} GB/s; "
        f"{value / 1e6:.1f} M tokens/s, {tflops:.1f} TFLOP/s; step bytes {step_bytes / 1e6:.0f} MB "
        f"-> {step_bytes / ms_per_step / 1e6:.0f} GB/s ({step_bytes / ms_per_step / 1e6 / HBM_PEAK_GBS:.1%} of HBM)")

    sweep = {}
    if args.sweep:
        for ww in (16, 32, 64, 128, 256, 512):
            for name in ("sa", "swa"):
                def run(s, ww=ww, name=name):
                    if name == "sa":
                        ssw.sa_forward(s["q"], s["k"], s["v"], s["sigma"], ww, True, out=s["out"])
                    else:
                        ssw.swa_forward(s["q"], s["k"], s["v"], ww, True, out=s["out"])
                for i in range(3):
                    run(sets[i % ROT])
                torch.cuda.synchronize()
                start.record(stream)
                for i in range(30):
                    run(sets[i % ROT])
                end.record(stream)
                torch.cuda.synchronize()
                t = start.elapsed_time(end) / 30
                byt = pass_bytes(B, n, Hq, Hkv, d, 2, sa=(name == "sa"), accumulate=False) - B * n * Hq * 4
                sweep[f"{name}_w{ww}_us"] = round(t * 1e3, 1)
                log(f"  {name.upper()} alone w={ww}: {t * 1e3:.1f} us, {n / t / 1e3:.1f} M tok/s, "
                    f"{byt / t / 1e6:.0f} GB/s, {4 * d * Hq * causal_pairs(n, ww) / t / 1e9:.1f} TFLOP/s")

    cpu = None
    if pool is not None:
        cpu = pool.baseline(args.cpu_rows)
        pool.close()

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q,K,V ~ N(0,1), gates sigmoid(N(0,1)), seeded sigma",
        "config": {"workload": f"{wl.name} gated SA+SWA forward", "B": B, "n": n, "Hq": Hq,
                   "Hkv": Hkv, "d": d, "window": w, "causal": causal},
        "tflops": round(tflops, 2),
        "tflops_frac_bf16": round(tflops / BF16_PEAK_TFLOPS, 4),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "passes_us": {"sa_pass": round(sa_ms * 1e3, 1), "swa_pass": round(swa_ms * 1e3, 1),
                      "dispatches_timed": len(quads),
                      "step_first_quarter": round(span_first * 1e3, 1),
                      "step_last_quarter": round(span_last * 1e3, 1)},
        "sigma_host_ms": round(sigma_ms, 2),
        "copy_gbs": round(copy_gbs, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if sweep:
        line["sweep_us"] = sweep
    print(json.dumps(line), flush=True)


def nsweep(args):
    """SA (causal, w = --window) against full causal attention on the same kernels (the SWA kernel
    with a window covering the sequence), layer shape of the long-context workload (32 query / 8 KV
    heads, d 128, bf16), n = 2048 .. 32768.  Prints one JSON line with per-n times and the ratio."""
    import numpy as np
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w = args.window
    B, Hq, Hkv, d = 1, 32, 8, 128
    rows = []
    for n in (2048, 4096, 8192, 16384, 32768):
        q, k, v = synth.qkv(synth.data_seed(4, 0), B, n, Hq, Hkv, d, "bf16")
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        sigma = torch.from_numpy(ssw.make_permutation(synth.sigma_seed(4, 0), n)).to(dev)
        out = torch.empty_like(q)

        def timed(fn, reps):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(reps):
                fn()
            end.record(stream)
            torch.cuda.synchronize()
            return start.elapsed_time(end) / reps

        t_sa = timed(lambda: ssw.sa_forward(q, k, v, sigma, w, True, out=out), 20)
        t_full = timed(lambda: ssw.swa_forward(q, k, v, n, True, out=out), 3 if n >= 16384 else 10)
        full_flops = 4 * d * B * Hq * (n * (n + 1) // 2)
        sa_flops = 4 * d * B * Hq * causal_pairs(n, w)
        row = {"n": n, "sa_us": round(t_sa * 1e3, 1), "full_us": round(t_full * 1e3, 1),
               "full_over_sa": round(t_full / t_sa, 2),
               "sa_tflops": round(sa_flops / (t_sa * 1e-3) / 1e12, 1),
               "full_tflops": round(full_flops / (t_full * 1e-3) / 1e12, 1)}
        log(f"n={n}: SA w={w} {row['sa_us']} us, full causal {row['full_us']} us, "
            f"ratio {row['full_over_sa']}x; full attention {row['full_tflops']} TFLOP/s "
            f"({row['full_tflops'] / BF16_PEAK_TFLOPS:.1%} of bf16 MFMA peak)")
        rows.append(row)
        del q, k, v, out
    line = {"metric": "full causal attention time / SA time (same kernels), 1 GPU",
            "unit": "ratio", "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "long-context layer shape, n sweep", "B": B, "Hq": Hq,
                       "Hkv": Hkv, "d": d, "window": w, "causal": True},
            "sweep": rows}
    print(json.dumps(line), flush=True)


def train(args):
    """The gated layer's training step at the long-context workload (B 1, n 32768, 32 / 8 heads,
    d 128, bf16, causal, w = --window): ssw_gated_sa_swa_forward_train (SWA and SA passes with
    lse, gate combine) then ssw_gated_sa_swa_backward (dQ and dK/dV kernels for each path).
    Also times the backward alone and each path's backward alone.  One JSON line."""
    import numpy as np
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    wl = synth.workload(4)
    B, n, Hq, Hkv, d = wl.B, wl.n, wl.Hq, wl.Hkv, wl.d
    w = args.window
    causal = True
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    seed = synth.data_seed(4, 0)
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, wl.dtype)
    g = synth.gates(seed, B, n, Hq)
    dy = synth.upstream_grad(seed, B, n, Hq, d, wl.dtype)
    sigma = ssw.make_permutation(synth.sigma_seed(4, 0), n)
    ROT = 2
    sets = []
    for _ in range(ROT):
        s = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev), g=g.to(dev), dy=dy.to(dev),
                 sigma=torch.from_numpy(sigma).to(dev), out=torch.empty(B, n, Hq, d, dtype=q.dtype,
                                                                        device=dev))
        s["saved"] = ssw.gated_sa_swa_forward_train(s["q"], s["k"], s["v"], s["sigma"], w, causal,
                                                    s["g"], out=s["out"])[1]
        s["grads"] = ssw.gated_sa_swa_backward(s["q"], s["k"], s["v"], s["sigma"], w, causal,
                                               s["g"], s["saved"], s["dy"])
        s["delta"] = torch.empty(B, n, Hq, dtype=torch.float32, device=dev)
        sets.append(s)
    torch.cuda.synchronize()

    def fwd(s):
        ssw.gated_sa_swa_forward_train(s["q"], s["k"], s["v"], s["sigma"], w, causal, s["g"],
                                       out=s["out"], saved=s["saved"])

    def bwd(s):
        dq, dk, dv, dg = s["grads"]
        ssw.gated_sa_swa_backward(s["q"], s["k"], s["v"], s["sigma"], w, causal, s["g"],
                                  s["saved"], s["dy"], dq=dq, dk=dk, dv=dv, dgates=dg,
                                  delta=s["delta"])

    def path_bwd(s, sa):
        dq, dk, dv, dg = s["grads"]
        y_sa, lse_sa, y_swa, lse_swa = s["saved"]
        if sa:
            ssw.sa_backward(s["q"], s["k"], s["v"], s["sigma"], w, causal, y_sa, lse_sa, s["dy"],
                            gate=s["g"][0], dq=dq, dk=dk, dv=dv, dgate=dg[0], delta=s["delta"])
        else:
            ssw.swa_backward(s["q"], s["k"], s["v"], w, causal, y_swa, lse_swa, s["dy"],
                             gate=s["g"][1], dq=dq, dk=dk, dv=dv, dgate=dg[1], delta=s["delta"])

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed(fn, K, W):
        for i in range(W):
            fn(sets[i % ROT])
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            fn(sets[i % ROT])
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    K, W = args.steps, args.warmup
    step_ms = timed(lambda s: (fwd(s), bwd(s)), K, W)
    fwd_ms = timed(fwd, K, W)
    bwd_ms = timed(bwd, K, W)
    sa_bwd_ms = timed(lambda s: path_bwd(s, True), K, W)
    swa_bwd_ms = timed(lambda s: path_bwd(s, False), K, W)

    pairs = causal_pairs(n, w)
    fwd_flops = 2 * 4 * d * B * Hq * pairs          # two paths, QK^T and PV
    bwd_flops = 2 * 10 * d * B * Hq * pairs         # two paths, S, dP, dV, dK, dQ
    e = 2
    big, small, rows = B * n * Hq * d * e, B * n * Hkv * d * e, B * n * Hq * 4
    # one path's backward: q, k, v, A, dy, lse, gate (+ sigma) read; dq, dk, dv, dgate written
    path_bytes = 3 * big + 2 * small + 2 * rows + big + 2 * small + rows
    bwd_bytes = 2 * path_bytes + big + 2 * small     # the second path adds to dq, dk, dv
    tokens = B * n
    line = {
        "metric": "gated SA+SWA training step (fwd with lse + bwd) tokens/s at n=32K, w=128 (1 GPU)",
        "value": round(tokens / (step_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic: Q,K,V,dY ~ N(0,1), gates sigmoid(N(0,1)), seeded sigma",
        "config": {"workload": f"{wl.name} gated SA+SWA training step", "B": B, "n": n, "Hq": Hq,
                   "Hkv": Hkv, "d": d, "window": w, "causal": causal},
        "fwd_train_us": round(fwd_ms * 1e3, 1), "bwd_us": round(bwd_ms * 1e3, 1),
        "sa_bwd_us": round(sa_bwd_ms * 1e3, 1), "swa_bwd_us": round(swa_bwd_ms * 1e3, 1),
        "step_tflops": round((fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
        "bwd_algorithmic_bytes": bwd_bytes,
        "bwd_hbm_gbs": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1),
    }
    log(f"training step {step_ms * 1e3:.1f} us: forward {fwd_ms * 1e3:.1f} us, backward "
        f"{bwd_ms * 1e3:.1f} us (SA path {sa_bwd_ms * 1e3:.1f}, SWA path {swa_bwd_ms * 1e3:.1f}); "
        f"backward {line['bwd_tflops']} TFLOP/s, {line['bwd_hbm_gbs']} GB/s algorithmic")
    print(json.dumps(line), flush=True)


def all_configs(args):
    """Every synthetic workload (synth.WORKLOADS) on its own paths and windows: per layer time,
    tokens/s, algorithmic TFLOP/s and the fraction of the HBM roofline (algorithmic bytes of the
    passes: each operand read once, outputs written once; the gated layer's two passes include
    the intermediate write and read).  Each layer draws its own sigma; the Q/K/V draw of layer 0
    is reused for the timing of every layer."""
    import numpy as np
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    rows = []
    for wl in synth.WORKLOADS:
        B, n, Hq, Hkv, d = wl.B, wl.n, wl.Hq, wl.Hkv, wl.d
        elem = 4 if wl.dtype == "f32" else 2
        q, k, v = synth.qkv(synth.data_seed(wl.index, 0), B, n, Hq, Hkv, d, wl.dtype)
        g = synth.gates(synth.data_seed(wl.index, 0), B, n, Hq)
        q, k, v, g = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
        out = torch.empty_like(q)
        sigmas = [torch.from_numpy(ssw.make_permutation(synth.sigma_seed(wl.index, l), n)).to(dev)
                  for l in range(wl.layers)]
        reps = 200 if n * B <= 8192 else 20
        for w in wl.windows:
            for causal in wl.causal_modes:
                for path in wl.paths:
                    ts = []
                    for sg in sigmas:
                        if path == "sa":
                            fn = lambda sg=sg: ssw.sa_forward(q, k, v, sg, w, causal, out=out)
                        elif path == "swa":
                            fn = lambda: ssw.swa_forward(q, k, v, w, causal, out=out)
                        else:
                            fn = lambda sg=sg: ssw.gated_sa_swa_forward(q, k, v, sg, w, causal, g,
                                                                        out=out)
                        ts.append(timed(fn, reps))
                        if path == "swa":
                            break  # no sigma: every layer is the same computation
                    t = float(np.mean(ts))
                    ww = min(w, n)
                    pairs = causal_pairs(n, ww) if causal else n * (2 * ww - 1) - ww * (ww - 1)
                    npath = 2 if path == "gated" else 1
                    flops = npath * 4 * d * B * Hq * pairs
                    if path == "gated":
                        byt = (pass_bytes(B, n, Hq, Hkv, d, elem, sa=False, accumulate=False) +
                               pass_bytes(B, n, Hq, Hkv, d, elem, sa=True, accumulate=True))
                    else:
                        byt = pass_bytes(B, n, Hq, Hkv, d, elem, sa=(path == "sa"),
                                         accumulate=False) - B * n * Hq * 4
                    gbs = byt / (t * 1e-3) / 1e9
                    row = {"workload": wl.name, "path": path, "window": w, "causal": causal,
                           "dtype": wl.dtype, "layers_timed": len(ts),
                           "us_per_layer": round(t * 1e3, 2),
                           "tokens_per_s": round(B * n / (t * 1e-3), 1),
                           "tflops": round(flops / (t * 1e-3) / 1e12, 2),
                           "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
                    log(f"{wl.name} {path} w={w} causal={causal}: {row['us_per_layer']} us/layer, "
                        f"{row['tokens_per_s'] / 1e6:.2f} M tok/s, {row['tflops']} TFLOP/s, "
                        f"{row['hbm_gbs']} GB/s ({row['hbm_frac']:.1%} of HBM)")
                    rows.append(row)
        del q, k, v, g, out, sigmas
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "per-workload layer throughput (1 GPU)", "unit": "tokens/s",
                      "higher_is_better": True, "data": "synthetic", "rows": rows}), flush=True)


def gates_bench(args):
    """ssw_gate_projection on the long-context layer's tokens: x [32768, 4096] bf16 (a hidden size
    of 4096), 32 query heads (64 outputs).  HBM roofline on x read once plus the gates written."""
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    rows, Hm, Hq = 32768, 4096, 32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    x, w_t, bias = synth.gate_inputs(synth.data_seed(4, 0), rows, Hm, Hq)
    xs = [x.to(dev) for _ in range(3)]  # rotated so no call finds x in the last-level cache
    w_t, bias = w_t.to(dev), bias.to(dev)
    out = torch.empty(2, rows, Hq, dtype=torch.float32, device=dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    for i in range(5):
        ssw.gate_projection(xs[i % 3], w_t, bias, out=out)
    torch.cuda.synchronize()
    K = 60
    start.record(stream)
    for i in range(K):
        ssw.gate_projection(xs[i % 3], w_t, bias, out=out)
    end.record(stream)
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / K
    byt = rows * Hm * 2 + 2 * Hq * Hm * 2 + 2 * rows * Hq * 4
    gbs = byt / (t * 1e-3) / 1e9
    line = {"metric": "gate projections sigmoid(x w + b) (1 GPU)", "unit": "us",
            "value": round(t * 1e3, 2), "higher_is_better": False, "dtype": "bf16",
            "data": "synthetic", "config": {"rows": rows, "Hm": Hm, "Hq": Hq},
            "tflops": round(2 * rows * Hm * 2 * Hq / (t * 1e-3) / 1e12, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": byt}}
    log(f"gate projection {rows}x{Hm} -> 2x{Hq}: {t * 1e3:.1f} us, {gbs:.0f} GB/s")
    print(json.dumps(line), flush=True)


def decode(args):
    """One gated decode step per batch row (ssw_gated_sa_swa_decode) over a KV cache of the
    long-context layer shape (32 query / 8 KV heads, d 128, bf16), n_max 32768, w = --window,
    batch --batch, positions drawn uniformly in [n_max / 2, n_max).  Also SA and SWA steps alone.
    The roofline counts the K/V rows each step must read: the SA neighbours (tokens <= t in the
    band of sigma^-1(t)) and the SWA window, plus q, out and the gates."""
    import numpy as np
    import torch

    import stochastic_sliding_window_amd as ssw
    import synth

    B, n, Hq, Hkv, d, w = args.batch, 32768, 32, 8, 128, args.window
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    seed = synth.data_seed(4, 0)
    rng = np.random.default_rng(seed)
    pos = rng.integers(n // 2, n, size=B).astype(np.int32)
    # the new tokens' queries; eight distinct caches drawn on the host, copied round-robin into
    # the B batch rows' own cache buffers on the device (each row still reads its own memory)
    q = synth.qkv(seed, B, 1, Hq, Hkv, d, "bf16")[0][:, 0].contiguous()
    kd = torch.empty(B, n, Hkv, d, dtype=torch.bfloat16, device=dev)
    vd = torch.empty_like(kd)
    for i in range(min(B, 8)):
        _, kb, vb = synth.qkv(seed + 1 + i, 1, n, 1, Hkv, d, "bf16")
        kb, vb = kb[0].to(dev), vb[0].to(dev)
        for b in range(i, B, 8):
            kd[b].copy_(kb)
            vd[b].copy_(vb)
    log(f"decode caches ready: {B} rows of {n} positions")
    g = synth.gates(seed, B, 1, Hq)[:, :, 0].contiguous()
    sig, inv = ssw.make_permutation(synth.sigma_seed(4, 0), n, with_inverse=True)
    qd, gd = q.to(dev), g.to(dev)
    sd, invd, posd = (torch.from_numpy(x).to(dev) for x in (sig, inv, pos))
    out = torch.empty_like(qd)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed(fn, K=200, W=10):
        for _ in range(W):
            fn()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(K):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    t_gated = timed(lambda: ssw.gated_sa_swa_decode(qd, kd, vd, sd, invd, posd, w, gd, out=out))
    t_sa = timed(lambda: ssw.sa_decode(qd, kd, vd, sd, invd, posd, w, out=out))
    t_swa = timed(lambda: ssw.swa_decode(qd, kd, vd, posd, w, out=out))

    # K/V rows each step must read (per KV head): SA neighbours + SWA window
    ww = min(w, n)
    sa_rows = swa_rows = 0
    for t in pos.tolist():
        p = int(inv[t])
        band = sig[max(0, p - ww + 1):min(n, p + ww)]
        sa_rows += int((band <= t).sum())
        swa_rows += min(ww, t + 1)
    row = d * 2
    kv_bytes = lambda rows: 2 * rows * Hkv * row
    qo_bytes = 2 * B * Hq * row
    gated_bytes = kv_bytes(sa_rows + swa_rows) + qo_bytes + 2 * B * Hq * 4
    sa_bytes = kv_bytes(sa_rows) + qo_bytes
    swa_bytes = kv_bytes(swa_rows) + qo_bytes
    gbs = gated_bytes / (t_gated * 1e-3) / 1e9
    line = {
        "metric": "gated SA+SWA decode step tokens/s over a KV cache (n_max=32K, w=128, 1 GPU)",
        "value": round(B / (t_gated * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic: Q,K,V ~ N(0,1), gates sigmoid(N(0,1)), seeded sigma, positions "
                "uniform in [n_max/2, n_max)",
        "config": {"workload": "decode, long-context layer shape", "B": B, "n_max": n, "Hq": Hq,
                   "Hkv": Hkv, "d": d, "window": w},
        "us_per_step": round(t_gated * 1e3, 2), "sa_us": round(t_sa * 1e3, 2),
        "swa_us": round(t_swa * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": gated_bytes},
        "sa_gbs": round(sa_bytes / (t_sa * 1e-3) / 1e9, 1),
        "swa_gbs": round(swa_bytes / (t_swa * 1e-3) / 1e9, 1),
        "mean_sa_neighbours": round(sa_rows / B, 1),
    }
    log(f"decode B={B}: gated {t_gated * 1e3:.1f} us ({gbs:.0f} GB/s), SA {t_sa * 1e3:.1f} us, "
        f"SWA {t_swa * 1e3:.1f} us; {sa_rows / B:.1f} SA neighbours per token")
    print(json.dumps(line), flush=True)


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE counter runs
    (scaled by the plain-copy calibration), or None when the kernel source has changed since the
    counters were taken (or no counters were taken for it)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_n32768_w128.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources_hashed"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["kernel_sha256"]:
        log(f"counter figures in {os.path.basename(path)} are for an older kernel: traffic = null")
        return None
    return rec["traffic_bytes_per_launch"]


def copy_bandwidth(dev, stream, start, end, nbytes=COPY_BYTES, reps=10):
    """Read+write GB/s of a plain elementwise copy (int32 negate) of `nbytes` HBM-resident bytes.

    Context for the roofline (what a streaming kernel reaches on this device), and the known-size
    kernel that scales the FETCH_SIZE / WRITE_SIZE counters in profiled runs."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        torch.neg(src, out=dst)
    end.record(stream)
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / reps
    gbs = 2 * nbytes / (t * 1e-3) / 1e9
    log(f"plain copy of {nbytes >> 20} MiB: {t * 1e3:.1f} us -> {gbs:.0f} GB/s (read + write)")
    del src, dst
    return gbs


# ---- the CPU oracle baseline, on every host core the process may use

_POOL_DATA = None


def _oracle_rows(rows):
    """Worker: the oracle's gated forward on the given query rows; returns the seconds taken."""
    import oracle
    from threadpoolctl import threadpool_limits
    qe, ke, ve, ge, sigma, w, causal = _POOL_DATA
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.gated_forward(qe, ke, ve, sigma, w, causal, ge, rows)
        return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class OraclePool:
    """The fp64 oracle, untuned, on a bounded sample of query rows of the same layer (both paths),
    split over one single-threaded worker process per available core (at most 16).  The workers
    are forked before the parent initialises the GPU and never touch it."""

    def __init__(self, q, k, v, g, sigma, w, causal):
        import multiprocessing as mp
        global _POOL_DATA
        self.avail = len(os.sched_getaffinity(0))
        self.workers = max(1, min(16, self.avail))
        self.n = q.shape[1]
        self.hq = q.shape[2]
        # exact float32 copies, shared with the forked workers copy-on-write
        _POOL_DATA = (q.float().numpy(), k.float().numpy(), v.float().numpy(), g.double().numpy(),
                      sigma, w, causal)
        self.pool = mp.get_context("fork").Pool(self.workers)

    def baseline(self, rows_req):
        import numpy as np
        rng = np.random.default_rng(0)
        n = self.n
        # one-off set-up in every worker, then a probe that sizes the sample to about 12 s
        self.pool.map(_oracle_rows, [rng.choice(n, size=4, replace=False)
                                     for _ in range(self.workers)])
        t_probe = _oracle_rows_probe(self.pool, rng, n, self.workers)
        rows = rows_req or max(64 * self.workers,
                               min(n, int(12.0 * self.workers / max(t_probe, 1e-6))))
        sample = rng.choice(n, size=rows, replace=False)
        t0 = time.perf_counter()
        self.pool.map(_oracle_rows, np.array_split(sample, 4 * self.workers))
        t = time.perf_counter() - t0
        tps = rows / t
        model = _cpu_model()
        log(f"cpu oracle: {rows} rows in {t:.1f}s -> {tps:.1f} tokens/s ({self.workers} worker "
            f"processes of one thread each, {self.avail} cores available; {model})")
        return {"value": round(tps, 2), "unit": "tokens/s", "cores": self.workers,
                "cores_available": self.avail, "cpu_model": model, "kind": "oracle",
                "sample": f"{rows} random query rows of the same layer (all {self.hq} heads, SA "
                          f"and SWA paths, gated), fp64 NumPy, split over {self.workers} "
                          f"single-threaded processes, {t:.1f} s wall"}

    def close(self):
        self.pool.close()
        self.pool.join()


def _oracle_rows_probe(pool, rng, n, workers):
    """Seconds per row of one worker, from 32 rows per worker."""
    ts = pool.map(_oracle_rows, [rng.choice(n, size=32, replace=False) for _ in range(workers)])
    return float(sum(ts)) / (32 * workers)


if __name__ == "__main__":
    main()
