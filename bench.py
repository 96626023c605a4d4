"""Benchmark of the layer-sliding training step on one MI355X.

One "step" is one sf_slide_step over a batch of synthetic inputs: forward
through every layer with the next layer's bf16 weights streamed in from
pinned host memory, the backward in reverse order with each layer's fp32
gradients streamed out to pinned host slots (window of 2 layers resident).
The default workload is the largest one a single GPU runs: a slice of eight
~123B-shaped layers (hidden 12288, 96 query heads x 128 with 8 KV heads,
ffn 28672, batch 1 x seq 4096) cycled through the window, x and dy ~ N(0, 1)
in, no head; its host optimizer is off (fp32 master weights and moments of
the eight layers would take 133 GB of host memory), gradients still leave
every layer.  Smaller workloads (``--workload``) add the embedding, the fused
LinearCrossEntropy head and host Adam on every layer.

Printed (one JSON line): tokens/s per layer fwd+bwd of the sliding step
(value), MFMA utilisation of the resident layer kernels, copy/compute
overlap of the sliding engine, the roofline of the dominant kernel (timed
live with HIP events), and the fp64 oracle's CPU throughput on a bounded
sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBPS = 8000.0


def time_gemms(w, sf, torch, reps=20):
    """Average duration (ms) of each layer GEMM, launched alone on the current stream."""
    from layer_sliding_offloaded_amd import runtime as rt
    dt, tdt = rt.sf_dtype(w), rt.storage_dtype(w)
    s = torch.cuda.current_stream()
    out = {}
    from layer_sliding_offloaded_amd.prof import layer_gemms
    for name, lay, M, N, K in layer_gemms(w):
        a_shape = (K, M) if lay == 2 else (M, K)
        b_shape = (N, K) if lay == 0 else (K, N)
        A = torch.randn(a_shape, device="cuda").to(tdt)
        B = torch.randn(b_shape, device="cuda").to(tdt)
        C = torch.empty((M, N), device="cuda", dtype=torch.float32 if lay == 2 else tdt)
        f32out = 1 if lay == 2 else 0
        wsb = sf.sf_gemm_workspace_bytes(M, N, K)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        call = lambda: sf.sf_gemm(dt, lay, f32out, M, N, K, A.data_ptr(), a_shape[1], B.data_ptr(), b_shape[1],
                                  C.data_ptr(), N, s.cuda_stream, ws.data_ptr(), wsb)
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            call()
        e1.record(s)
        torch.cuda.synchronize()
        out[name] = dict(layout=lay, M=M, N=N, K=K, ms=e0.elapsed_time(e1) / reps)
        del A, B, C
    return out


def stored_traffic(workload, role):
    """HBM bytes per launch of a layer GEMM, from the committed rocprofv3
    counter summary (profiles/gemm_traffic_<workload>.md), or None when there
    is none or the GEMM source has changed since the counters were taken."""
    from layer_sliding_offloaded_amd import prof
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    sha, table = None, None
    with open(path) as fh:
        for line in fh:
            if line.startswith("gemm_source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("traffic_bytes:"):
                table = json.loads(line.split(":", 1)[1])
    if sha != prof.gemm_source_hash() or not table or role not in table:
        return None
    return table[role]


def link_probe(torch, nbytes=256 << 20, reps=4):
    """Pinned host <-> device copy rates (GB/s) measured with hipMemcpyAsync
    (torch copies of pinned buffers): each direction alone, then both at once
    on two streams of default priority."""
    h_src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h_dst = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d_dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d_src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s_up, s_down = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn, stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        return e0, e1

    def rate(e):
        return nbytes * reps / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9

    up = lambda: [d_dst.copy_(h_src, non_blocking=True) for _ in range(reps)]
    down = lambda: [h_dst.copy_(d_src, non_blocking=True) for _ in range(reps)]
    with torch.cuda.stream(s_up):
        up()  # warm-up
        eu = timed(up, s_up)
    torch.cuda.synchronize()
    with torch.cuda.stream(s_down):
        down()
        ed = timed(down, s_down)
    torch.cuda.synchronize()
    with torch.cuda.stream(s_up):
        bu = timed(up, s_up)
    with torch.cuda.stream(s_down):
        bd = timed(down, s_down)
    torch.cuda.synchronize()
    out = {"h2d_gbps": round(rate(eu), 2), "d2h_gbps": round(rate(ed), 2),
           "bidir_h2d_gbps": round(rate(bu), 2), "bidir_d2h_gbps": round(rate(bd), 2),
           "probe": f"{reps} x {nbytes >> 20} MiB pinned copies per direction"}
    del h_src, h_dst, d_dst, d_src
    return out


def cpu_baseline(w, target_s=12.0):
    """The fp64 oracle, as it stands, on one layer fwd+bwd of a bounded slice
    (batch 1) of the workload, repeated until about target_s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import seeded_inputs as si

    # batch 1, and a sequence prefix short enough for ~1.5 TFLOP of fp64 work per repetition
    p_lin = (w.n_heads + 2 * w.n_kv_heads) * w.head_dim * w.hidden + w.hidden * w.n_heads * w.head_dim \
        + 3 * w.ffn * w.hidden
    seq = min(w.seq, max(64, int(1.5e12 / (6.0 * p_lin)) // 64 * 64))
    ws = w.with_(batch=1, seq=seq)
    p = {k: v.astype(np.float64) for k, v in si.layer_params(ws, 0).items()}
    x = si.layer_input(ws).astype(np.float64)
    dy = si.upstream_grad(ws).astype(np.float64)
    sh = oracle.LayerShape(ws.hidden, ws.n_heads, ws.n_kv_heads, ws.head_dim, ws.ffn, ws.batch, ws.seq, ws.eps,
                           ws.rope_base)
    n = 0
    t0 = time.perf_counter()
    while True:
        y, cache = oracle.layer_fwd(p, x, sh)
        oracle.layer_bwd(p, cache, dy, sh)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s or n >= 1000:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(n * ws.tokens / el, 2), "unit": "tokens/s per layer (fwd+bwd)", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} x one layer fwd+bwd, fp64 numpy, batch 1 x seq {ws.seq}, hidden {ws.hidden} "
                      f"({el:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # default 20 steps at the 123B-shaped slice (~25 s timed), 50 elsewhere
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="slice123b-gqa-bf16")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default=None,
                    help="16-bit storage type (default: the workload's); f16 runs with dynamic loss scaling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--adam-threads", type=int, default=0)
    ap.add_argument("--trace", default=None,
                    help="write the last timed step's engine timeline (kind, start_ms, end_ms, info) as CSV")
    ap.add_argument("--no-adam", action="store_true",
                    help="stream gradients out but skip the optimizer (default for the 123B-shaped slice, whose "
                         "fp32 Adam states would need 133 GB of host memory)")
    ap.add_argument("--grad-slots", type=int, default=2,
                    help="pinned fp32 gradient slots shared by all layers (a ring; n_layers = one buffer per layer)")
    ap.add_argument("--sync", "--sync-adam", dest="sync", action="store_true",
                    help="every step waits for its own host Adam and copies before returning (default: pipelined "
                         "steps: host Adam, or without Adam the last gradient copies, run on into the next step, "
                         "whose forward waits per layer for what it reads)")
    ap.add_argument("--no-keep", action="store_true",
                    help="without Adam, upload layers 0..window-1 again in every forward (default: they stay in "
                         "their units from the previous backward)")
    ap.add_argument("--ckpt", action="store_true",
                    help="sliding activation checkpointing: layer inputs wait in pinned host memory and each "
                         "layer's forward is recomputed before its backward")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported: the layer-sliding step is a "
              "single-GPU method and this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import seeded_inputs as si
    from layer_sliding_offloaded_amd import runtime as rt
    from layer_sliding_offloaded_amd import sf

    from layer_sliding_offloaded_amd.prof import layer_flops

    sf.load()
    torch.cuda.set_device(0)
    w = si.WORKLOADS[args.workload]
    if args.layers:
        w = w.with_(n_layers=args.layers)
    big = w.name == "slice123b-gqa-bf16"
    if args.dtype and args.dtype != w.dtype:
        if w.dtype == "f32":
            sys.exit(f"--dtype: {w.name} is an fp32 workload")
        w = w.with_(dtype=args.dtype, name=w.name.rsplit("-", 1)[0] + "-" + args.dtype)
    if args.steps is None:
        args.steps = 20 if big else 50
    if args.warmup is None:
        args.warmup = 2 if big else 5
    print(f"[bench] workload {w}", file=sys.stderr, flush=True)

    adam = not args.no_adam and not big
    t_setup = time.perf_counter()
    kept = {}

    def draw(l):
        p = si.layer_params(w, l)
        if l == 0:
            kept[0] = p  # for the resident-layer measurement
        print(f"[bench] layer {l} parameters drawn ({time.perf_counter() - t_setup:.1f} s)", file=sys.stderr,
              flush=True)
        return p

    head = None
    if w.vocab:
        head = dict(E=si.embedding(w), gf=si.final_gain(w), Wlm=si.lm_head(w))
    # pipelined: host Adam, or without Adam a step's last gradient copies,
    # run on into the next step.  Without Adam the parameters never change,
    # so the layers that end the backward in their units also open the next
    # forward (keep-turnaround)
    pipeline = not args.sync
    keep = not adam and not args.no_keep
    # draws run on a few host threads (each layer has its own seed)
    ncpu = len(os.sched_getaffinity(0))
    eng = rt.Engine(w, draw, head, window=w.window, n_grad_slots=args.grad_slots, adam=adam, chunk=2048,
                    adam_threads=args.adam_threads, ckpt=args.ckpt, pipeline=pipeline, keep_turnaround=keep,
                    draw_threads=max(1, min(8, ncpu // 2)))
    hbm = {"unit_pool_bytes": eng.pool.numel(), "activation_bytes": eng.act_bytes}
    # host memory the engine holds for the layers (pinned: bf16 params, fp32
    # gradient slots, checkpoints; pageable: fp32 master weights and moments)
    host = {"params_pinned": sum(t.numel() for t in eng.h_params),
            "grad_slots_pinned": sum(t.numel() for t in eng.h_slots),
            "checkpoints_pinned": eng.h_ckpt.numel() if eng.h_ckpt is not None else 0,
            "master_m_v": sum(3 * m.nbytes for m in eng.h_master)}
    host["total"] = sum(host.values())
    host["grad_slots"] = args.grad_slots
    print(f"[bench] engine ready ({time.perf_counter() - t_setup:.1f} s)", file=sys.stderr, flush=True)
    if head is not None:
        d_in = torch.from_numpy(si.token_ids(w).reshape(-1)).cuda()
        d_dy = None
    else:
        d_in = rt.to_storage_tensor(si.layer_input(w), w).cuda()
        d_dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()
    for i in range(args.warmup):
        loss, st = eng.step(d_in, d_dy)
        print(f"[bench] warmup {i} loss {loss:.4f} wall {st['wall_ms']:.2f} ms", file=sys.stderr, flush=True)
    eng.sync()
    torch.cuda.synchronize()
    stats = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        loss, st = eng.step(d_in, d_dy)
        stats.append(st)
    # the last steps' Adam and uploads belong to the timed work
    agg = eng.sync()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1000.0 * elapsed / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step"
          + (f", loss {loss:.4f}" if head is not None else " (no head: no loss)"), file=sys.stderr, flush=True)
    if pipeline:
        # one measurement window over the timed steps: per-step means of times
        # and bytes; rates and the overlap share over the whole window
        per_step = ("compute_ms", "copy_ms", "h2d_ms", "d2h_ms", "busy_ms", "span_ms", "adam_ms", "h2d_bytes",
                    "d2h_bytes")
        med = {k: (v / args.steps if k in per_step else v) for k, v in agg.items()}
        med["wall_ms"] = float(np.median([s["wall_ms"] for s in stats]))
        med["loss"] = float(loss)
    else:
        med = {k: float(np.median([s[k] for s in stats])) for k in stats[0]}
    if args.trace:
        with open(args.trace, "w") as f:
            f.write("kind,start_ms,end_ms,info\n")
            for k, a, b, x in eng.trace():
                f.write(f"{k},{a:.4f},{b:.4f},{x:.0f}\n")
    eng.close()
    del eng

    # resident layer kernels: one layer fwd + bwd with weights in HBM
    p = kept.pop(0)
    c = rt.Context(w, 2048)
    L = c.layout
    dw = rt.pack_params(L, p, w).cuda()
    x = rt.to_storage_tensor(si.layer_input(w), w).cuda()
    dy = rt.to_storage_tensor(si.upstream_grad(w), w).cuda()
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    saved = rt.device_bytes(L.saved_bytes)
    g = torch.empty(L.grad_bytes // 4, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def layer_step():
        sf.sf_layer_fwd(c.ctx, dw.data_ptr(), x.data_ptr(), y.data_ptr(), saved.data_ptr(), s.cuda_stream)
        sf.sf_layer_bwd(c.ctx, dw.data_ptr(), x.data_ptr(), saved.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                        g.data_ptr(), s.cuda_stream)

    for _ in range(3):
        layer_step()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        layer_step()
    e1.record(s)
    torch.cuda.synchronize()
    layer_ms = e0.elapsed_time(e1) / reps
    fl = layer_flops(w)
    peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS  # fp16 MFMA: the bf16 rate
    layer_tflops = fl / (layer_ms * 1e-3) / 1e12
    c.close()
    del dw, x, dy, y, dx, saved, g

    # dominant kernel: the layer GEMM with the longest launch, timed alone
    gem = time_gemms(w, sf, torch)
    dom_name = max(gem, key=lambda k: gem[k]["ms"])
    dom = gem[dom_name]
    dom_flops = 2.0 * dom["M"] * dom["N"] * dom["K"]
    achieved = dom_flops / (dom["ms"] * 1e-3) / 1e12
    print(f"[bench] layer fwd+bwd {layer_ms:.3f} ms ({layer_tflops:.1f} TFLOP/s); GEMMs: "
          + ", ".join(f"{k} {v['ms']:.3f}ms" for k, v in gem.items()), file=sys.stderr, flush=True)

    T = w.tokens
    value = T * w.n_layers / (ms_step * 1e-3)
    out = {
        "metric": "train tokens/s per layer fwd+bwd (bf16) at 1 GPU; MFMA util %; copy overlap %",
        "value": round(value, 1),
        "unit": "tokens/s per layer (fwd+bwd)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_layers": w.n_layers, "window": w.window, "batch": w.batch,
                   "seq": w.seq, "hidden": w.hidden, "heads": w.n_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "ffn": w.ffn, "vocab": w.vocab,
                   "adam": ("host fp32 (layers), device fp32 (resident embedding/head)" if adam else "off"),
                   "activation_checkpointing": args.ckpt,
                   "adam_schedule": ("pipelined across steps" if pipeline else "synchronous per step") if adam
                   else "off",
                   "step_schedule": "pipelined across steps" if pipeline else "synchronous per step",
                   "turnaround_layers_kept": keep,
                   "parallelism": "none (1 GPU)"},
        "engine_hbm": hbm,
        "engine_host_bytes": host,
        "mfma_util_pct": round(100.0 * layer_tflops / peak, 2),
        "kernel_tokens_per_s_per_layer": round(T / (layer_ms * 1e-3), 1),
        "layer_fwd_bwd_ms": round(layer_ms, 4),
        "overlap_pct": round(med["overlap_pct"], 2),
        "engine": {k: round(v, 4) for k, v in med.items()},
        "gemm_ms": {k: round(v["ms"], 5) for k, v in gem.items()},
        "roofline": {"bound": "mfma", "kernel": f"gemm {dom_name} ({['NT', 'NN', 'TN'][dom['layout']]}, "
                                                f"M={dom['M']} N={dom['N']} K={dom['K']})",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": stored_traffic(w.name, dom_name)},
    }
    # host-link roofline: the step's bytes each way at the probe's rate for
    # that direction alone (the link is full duplex; the probe's rates with
    # both directions at once are reported too, but steps have exceeded them)
    link = link_probe(torch)
    t_link = max(med["h2d_bytes"] / (link["h2d_gbps"] * 1e9), med["d2h_bytes"] / (link["d2h_gbps"] * 1e9))
    link_tok = T * w.n_layers / t_link if t_link > 0 else None
    out["host_link"] = dict(link, step_h2d_gbps=round(med["h2d_gbps"], 2), step_d2h_gbps=round(med["d2h_gbps"], 2),
                            link_bound_tokens_per_s_per_layer=round(link_tok, 1) if link_tok else None,
                            frac=round(value / link_tok, 4) if link_tok else None)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
