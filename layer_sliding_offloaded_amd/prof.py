"""Profiling helpers: HBM traffic of the layer GEMMs from rocprofv3 counters,
and per-kernel duration summaries of a rocprofv3 kernel trace.

Modes:

* ``probe``: run, once each after a warm-up, a plain device copy of a known
  size (the calibration kernel) and then every layer GEMM of a workload,
  launched alone through ``sf_gemm`` exactly as ``bench.py`` times them.
  Meant to run under ``rocprofv3 --pmc FETCH_SIZE`` and, separately,
  ``rocprofv3 --pmc WRITE_SIZE``.
* ``summarize``: read the two counter CSVs, scale each GEMM's counter by
  (copy bytes / copy counter) -- the factor that turns the counter into
  bytes on this machine -- and print a markdown table plus the
  machine-readable lines ``bench.py`` reads.
* ``kernels``: per (kernel, grid) launch count, total and average duration
  from a rocprofv3 ``--kernel-trace`` database (``*_results.db``).
* ``gemm-runs``: from the same database, the average duration of each layer
  GEMM in ``bench.py``'s own per-GEMM timing loop (to set against the
  durations ``bench.py`` measures with HIP events).
* ``rowops``: from a kernel trace of ``bench.py``, the HBM-bound kernels of
  the layer and head (RMSNorm forward / backward, gain-gradient partials,
  the attention-backward row dot, cross-entropy rows, embedding gather, the
  device Adam of the embedding / LM head): median duration, algorithmic
  bytes per launch for the workload, achieved GB/s and the fraction of the
  8 TB/s HBM peak.  The median is taken over all launches; most of them are
  bench.py's resident-layer loop, where nothing else runs.
* ``layer-probe``: the ``probe`` sequence (calibration copy, then the 12
  layer GEMMs through ``sf_gemm``) followed by one resident decoder layer
  forward + backward (``sf_layer_fwd`` / ``sf_layer_bwd``) at the workload's
  shape, each after a warm-up run.  Meant to run under ``rocprofv3 --pmc
  MfmaUtil MfmaFlopsBF16``.
* ``mfma``: from that counter CSV, per GEMM role and per kernel of the layer:
  MFMA busy share (``MfmaUtil``: SQ_VALU_MFMA_BUSY_CYCLES over active cycles
  of all SIMDs) and the bf16 MFMA FLOPs the hardware executed
  (``MfmaFlopsBF16``) against the algorithmic FLOPs.
* ``timeline``: from the engine timeline ``bench.py --trace`` writes (one
  row per timed interval: compute, H2D or D2H copy, host Adam), the busy
  time of each kind over the window, the gaps longer than ``--gap`` ms in
  which no D2H copy runs (with what the H2D copies and the kernels did
  meanwhile), and the busy share of each kind per ``--bucket`` ms.
* ``vendor``: each layer GEMM of a workload (or those named by ``--gemms``)
  through ``sf_gemm`` and through ``torch.mm`` (hipBLASLt), same operand
  layouts and output types, ``--reps`` launches of each after two warm-ups,
  timed with HIP events; prints both durations and TFLOP/s.  Under
  ``rocprofv3 --kernel-trace`` it also names the library's kernels.
* ``vendor-counters``: counter CSVs of ``rocprofv3 --pmc ... -- prof vendor``
  (same ``--workload``, ``--gemms`` and ``--reps``): per GEMM, every counter
  averaged over the timed launches of this library's kernel and of the
  library kernel, side by side.
* ``head-study``: the chunked LM head + cross-entropy (``sf_head_fwd_bwd``)
  at one shape for several chunk sizes, the largest being the whole token
  count (every logit materialised at once): device bytes of the head's
  workspace and of all its buffers, time per call and TFLOP/s.

    python -m layer_sliding_offloaded_amd.prof probe --workload stack4-h1024-bf16
    python -m layer_sliding_offloaded_amd.prof summarize FETCH_CSV WRITE_CSV --workload stack4-h1024-bf16
    python -m layer_sliding_offloaded_amd.prof kernels RESULTS_DB [--top N]
    python -m layer_sliding_offloaded_amd.prof gemm-runs RESULTS_DB --workload W
    python -m layer_sliding_offloaded_amd.prof rowops RESULTS_DB --workload W
    python -m layer_sliding_offloaded_amd.prof timeline TRACE_CSV [--gap 20] [--bucket 50]
    python -m layer_sliding_offloaded_amd.prof vendor --workload W [--gemms gu_fwd,o_fwd] [--reps 5]
    python -m layer_sliding_offloaded_amd.prof vendor-counters CSV... --workload W [--gemms ...] [--reps 5]
    python -m layer_sliding_offloaded_amd.prof head-study --hidden 4096 --vocab 128256 --batch 4 --seq 2048 \
        --chunks 8192,4096,2048,1024,512,256
"""

import argparse
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20


def gemm_source_hash():
    """sha256 of the GEMM kernel source with comments and blank lines
    removed: a stored traffic figure is valid only for that code."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm.h", "common.h"):
        with open(os.path.join(HERE, "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def layer_flops(w):
    """Algorithmic FLOPs of one layer forward + backward: 6 T P_lin + 6 B n_h S^2 d (causal half)."""
    T = w.tokens
    p_lin = (w.n_heads + 2 * w.n_kv_heads) * w.head_dim * w.hidden + w.hidden * w.n_heads * w.head_dim \
        + 3 * w.ffn * w.hidden
    attn = 6.0 * w.batch * w.n_heads * w.seq * w.seq * w.head_dim  # (2 fwd + 4 bwd) x 2 x S^2 d / 2
    return 6.0 * T * p_lin + attn


def layer_gemms(w):
    """The 12 GEMMs of one layer's forward + backward: (name, layout, M, N, K)."""
    T, H, F = w.tokens, w.hidden, w.ffn
    Nq = w.n_heads * w.head_dim
    Nqkv = (w.n_heads + 2 * w.n_kv_heads) * w.head_dim
    return [
        ("qkv_fwd", 0, T, Nqkv, H), ("o_fwd", 0, T, H, Nq), ("gu_fwd", 0, T, 2 * F, H), ("down_fwd", 0, T, H, F),
        ("down_dx", 1, T, F, H), ("down_dw", 2, H, F, T), ("gu_dx", 1, T, H, 2 * F), ("gu_dw", 2, 2 * F, H, T),
        ("o_dx", 1, T, Nq, H), ("o_dw", 2, H, Nq, T), ("qkv_dx", 1, T, H, Nqkv), ("qkv_dw", 2, Nqkv, H, T),
    ]


def _gemms(workload):
    sys.path.insert(0, os.path.dirname(HERE))
    import seeded_inputs as si
    return layer_gemms(si.WORKLOADS[workload])


def probe(workload):
    import torch

    from layer_sliding_offloaded_amd import sf
    sf.load()
    s = torch.cuda.current_stream()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    calls = []
    for name, lay, M, N, K in _gemms(workload):
        a_shape = (K, M) if lay == 2 else (M, K)
        b_shape = (N, K) if lay == 0 else (K, N)
        A = torch.randn(a_shape, device="cuda").to(torch.bfloat16)
        B = torch.randn(b_shape, device="cuda").to(torch.bfloat16)
        C = torch.empty((M, N), device="cuda", dtype=torch.float32 if lay == 2 else torch.bfloat16)
        wsb = sf.sf_gemm_workspace_bytes(M, N, K)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        calls.append((name, (A, B, C, ws),
                      lambda A=A, B=B, C=C, ws=ws, lay=lay, M=M, N=N, K=K, a=a_shape, b=b_shape, wsb=wsb:
                      sf.sf_gemm(sf.SF_BF16, lay, 1 if lay == 2 else 0, M, N, K, A.data_ptr(), a[1], B.data_ptr(),
                                 b[1], C.data_ptr(), N, s.cuda_stream, ws.data_ptr(), wsb)))
    # warm-up (not counted by the summary: it takes the last launch of each kind)
    dst.copy_(src)
    for _, _, f in calls:
        f()
    torch.cuda.synchronize()
    print("probe: copy", flush=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    for name, _, f in calls:
        print("probe:", name, flush=True)
        f()
        torch.cuda.synchronize()


def layer_probe(workload):
    """Calibration copy + the 12 layer GEMMs, then one resident layer
    forward + backward (each sequence after a warm-up run)."""
    import torch

    sys.path.insert(0, os.path.dirname(HERE))
    import seeded_inputs as si
    from layer_sliding_offloaded_amd import runtime as rt
    from layer_sliding_offloaded_amd import sf
    sf.load()
    w = si.WORKLOADS[workload]
    c = rt.Context(w, 2048)
    L = c.layout
    gen = torch.Generator(device="cuda").manual_seed(5)
    dw = torch.empty(L.param_bytes // 2, dtype=torch.bfloat16, device="cuda")
    dw.normal_(0.0, 0.02, generator=gen)
    for k in (7, 8):  # gains 1
        dw[L.off[k] // 2:(L.off[k] + L.bytes[k]) // 2] = 1.0
    x = torch.randn(w.tokens, w.hidden, generator=gen, device="cuda").to(torch.bfloat16)
    dy = torch.randn(w.tokens, w.hidden, generator=gen, device="cuda").to(torch.bfloat16)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    saved = rt.device_bytes(L.saved_bytes)
    g = torch.empty(L.grad_bytes // 4, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def layer():
        sf.sf_layer_fwd(c.ctx, dw.data_ptr(), x.data_ptr(), y.data_ptr(), saved.data_ptr(), s)
        sf.sf_layer_bwd(c.ctx, dw.data_ptr(), x.data_ptr(), saved.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                        g.data_ptr(), s)

    layer()
    torch.cuda.synchronize()
    probe(workload)
    print("probe: layer", flush=True)
    layer()
    torch.cuda.synchronize()
    c.close()


def _counter_rows(path):
    """{dispatch id: (kernel name, {counter: value})} in dispatch order."""
    acc = {}
    for r in _rows(path):
        k = int(r["Dispatch_Id"])
        name, cs = acc.setdefault(k, (r["Kernel_Name"], {}))
        cs[r["Counter_Name"]] = cs.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [acc[k] for k in sorted(acc)]


def mfma(csv_path, workload):
    """MFMA busy share and hardware vs algorithmic FLOPs (see the module docstring)."""
    sys.path.insert(0, os.path.dirname(HERE))
    import seeded_inputs as si
    w = si.WORKLOADS[workload]
    d = _counter_rows(csv_path)
    # the last calibration copy splits the warm-up from the measured sequence
    idx = max(i for i, (n, _) in enumerate(d) if "copyBuffer" in n)
    rest = d[idx + 1:]
    gemms = layer_gemms(w)
    print("| GEMM | M x N x K | MfmaUtil % | MFMA FLOPs (bf16, hardware) | algorithmic 2MNK | ratio |")
    print("|---|---|---:|---:|---:|---:|")
    i = 0
    for name, lay, M, N, K in gemms:
        util, fl = 0.0, 0.0
        kname, cs = rest[i]
        i += 1
        util = cs.get("MfmaUtil", 0.0)
        fl = cs.get("MfmaFlopsBF16", 0.0)
        while i < len(rest) and "splitk_reduce" in rest[i][0]:
            i += 1
        alg = 2.0 * M * N * K
        print(f"| {name} | {M} x {N} x {K} | {util:.1f} | {fl / 1e9:.2f} G | {alg / 1e9:.2f} G | {fl / alg:.3f} |")
    layer = rest[i:]
    T, S, B = w.tokens, w.seq, w.batch
    attn_fwd = 4.0 * B * w.n_heads * S * S * w.head_dim / 2
    print()
    print("Kernels of one resident layer forward + backward, in launch order:")
    print()
    print("| # | kernel | MfmaUtil % | MFMA FLOPs (bf16, hardware) |")
    print("|---:|---|---:|---:|")
    tot = 0.0
    for j, (kname, cs) in enumerate(layer):
        fl = cs.get("MfmaFlopsBF16", 0.0)
        tot += fl
        print(f"| {j} | `{short_name(kname)[:90]}` | {cs.get('MfmaUtil', 0.0):.1f} | {fl / 1e9:.2f} G |")
    print()
    print(f"Layer total: {tot / 1e12:.3f} TFLOP of bf16 MFMA work executed; algorithmic "
          f"{layer_flops(w) / 1e12:.3f} TFLOP (6 T P_lin + 6 B n_h S^2 d); attention forward alone is "
          f"{attn_fwd / 1e9:.1f} GFLOP algorithmic (causal half).")


def _selected(workload, gemms):
    sel = set(gemms.split(",")) if gemms else None
    return [g for g in _gemms(workload) if sel is None or g[0] in sel]


def vendor(workload, gemms, reps):
    """This library's GEMMs against torch.mm (hipBLASLt), see the module docstring."""
    import torch

    from layer_sliding_offloaded_amd import sf
    sf.load()
    s = torch.cuda.current_stream()

    def timed(f):
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            f()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    print("| GEMM | layout | M x N x K | this library us | TFLOP/s | hipBLASLt us | TFLOP/s | library / ours |")
    print("|---|---|---|---:|---:|---:|---:|---:|")
    for name, lay, M, N, K in _selected(workload, gemms):
        a_shape = (K, M) if lay == 2 else (M, K)
        b_shape = (N, K) if lay == 0 else (K, N)
        A = torch.randn(a_shape, device="cuda").to(torch.bfloat16)
        B = torch.randn(b_shape, device="cuda").to(torch.bfloat16)
        C = torch.empty((M, N), device="cuda", dtype=torch.float32 if lay == 2 else torch.bfloat16)
        wsb = sf.sf_gemm_workspace_bytes(M, N, K)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        ours = timed(lambda: sf.sf_gemm(sf.SF_BF16, lay, 1 if lay == 2 else 0, M, N, K, A.data_ptr(), a_shape[1],
                                        B.data_ptr(), b_shape[1], C.data_ptr(), N, s.cuda_stream, ws.data_ptr(),
                                        wsb))
        if lay == 0:
            lib = timed(lambda: torch.mm(A, B.t()))
        elif lay == 1:
            lib = timed(lambda: torch.mm(A, B))
        else:
            lib = timed(lambda: torch.mm(A.t(), B, out_dtype=torch.float32))
        fl = 2.0 * M * N * K
        print(f"| {name} | {['NT', 'NN', 'TN'][lay]} | {M} x {N} x {K} | {ours:.1f} | {fl / ours / 1e6:.0f} | "
              f"{lib:.1f} | {fl / lib / 1e6:.0f} | {lib / ours:.3f} |", flush=True)
        del A, B, C, ws


def vendor_counters(paths, workload, gemms, reps):
    """Counters of ``vendor`` launches, this library's kernel beside hipBLASLt's (see the module docstring)."""
    runs = []  # [(kind, [(name, counters, dur_us)])] over all files, merged per dispatch
    per = {}
    for path in paths:
        for r in _rows(path):
            n = r["Kernel_Name"]
            kind = "ours" if "sf::" in n or "_ZN2sf" in n else ("lib" if "Cijk" in n else None)
            if kind is None or "splitk_reduce" in n:
                continue
            k = (path, int(r["Dispatch_Id"]))
            e = per.setdefault(k, [kind, n, {}, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3])
            e[2][r["Counter_Name"]] = e[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    sel = _selected(workload, gemms)
    per_file = {}
    for (path, d), e in sorted(per.items()):
        per_file.setdefault(path, []).append(e)
    counters, rows = [], {}
    for path, seq in per_file.items():
        # per GEMM: this library's launches, then the library's, each 2 warm-ups + reps
        i = 0
        for name, *_ in sel:
            for kind in ("ours", "lib"):
                grp = seq[i:i + 2 + reps]
                i += 2 + reps
                if len(grp) < 2 + reps or any(g[0] != kind for g in grp):
                    raise SystemExit(f"{path}: unexpected launch sequence at {name} {kind}")
                slot = rows.setdefault((name, kind), {"name": grp[-1][1], "dur": []})
                for c in grp[-1][2]:
                    if c not in counters:
                        counters.append(c)
                    slot[c] = sum(g[2][c] for g in grp[2:]) / reps
                slot["dur"] += [g[3] for g in grp[2:]]
    print("| GEMM | kernel | us (under counters) | " + " | ".join(counters) + " |")
    print("|---|---|---:|" + "---:|" * len(counters))
    for name, *_ in sel:
        for kind in ("ours", "lib"):
            r = rows[(name, kind)]
            kn = short_name(r["name"])[:70] if kind == "ours" else r["name"].split("_MT")[0][-40:] + " MT" + \
                r["name"].split("_MT")[1].split("_")[0] if "_MT" in r["name"] else r["name"][:70]
            print(f"| {name} | `{kn}` | {sum(r['dur']) / len(r['dur']):.1f} | " +
                  " | ".join(f"{r.get(c, float('nan')):.4g}" for c in counters) + " |")


def _rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _dispatches(path, counter):
    """[(kernel name, value)] in dispatch order for one counter (summed over its instances)."""
    acc = {}
    for r in _rows(path):
        if not r["Counter_Name"].startswith(counter):
            continue
        k = int(r["Dispatch_Id"])
        name, v = acc.get(k, (r["Kernel_Name"], 0.0))
        acc[k] = (name, v + float(r["Counter_Value"]))
    return [acc[k] for k in sorted(acc)]


def summarize(fetch_csv, write_csv, workload):
    gemms = _gemms(workload)
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = _dispatches(path, counter)
        # the measured pass ends the run: the calibration copy, then one
        # sf_gemm per role (a split-K launch is a GEMM kernel followed by its
        # reduction); the copy is the dispatch just before that GEMM run
        idx = len(d) - 1
        while idx >= 0 and ("gemm" in d[idx][0] or "splitk_reduce" in d[idx][0]):
            idx -= 1
        copy_kib = d[idx][1]
        factor = COPY_BYTES / (copy_kib * 1024.0) if copy_kib > 0 else float("nan")
        rest = d[idx + 1:]
        per_role, i = {}, 0
        for name, lay, M, N, K in gemms:
            if i >= len(rest):
                break
            kib = rest[i][1]
            i += 1
            while i < len(rest) and "splitk_reduce" in rest[i][0]:
                kib += rest[i][1]
                i += 1
            per_role[name] = kib
        out[counter] = (copy_kib, factor, per_role)
    fk, ff, fr = out["FETCH_SIZE"]
    wk, wf, wr = out["WRITE_SIZE"]
    print(f"calibration: {COPY_BYTES} B device copy reads FETCH_SIZE {fk:.0f} KiB (factor {ff:.4f}), "
          f"WRITE_SIZE {wk:.0f} KiB (factor {wf:.4f})")
    print()
    print("| GEMM | layout | M x N x K | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | "
          "algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|---|")
    traffic = {}
    for name, lay, M, N, K in gemms:
        if name not in fr or name not in wr:
            continue
        b = fr[name] * 1024 * ff + wr[name] * 1024 * wf
        outb = 4 if lay == 2 else 2
        alg = 2 * (M * K + N * K) + outb * M * N
        traffic[name] = round(b)
        print(f"| {name} | {'NT NN TN'.split()[lay]} | {M} x {N} x {K} | {fr[name]:.0f} | {wr[name]:.0f} | "
              f"{b / 1e6:.1f} MB | {alg / 1e6:.1f} MB | {b / alg:.2f} |")
    print()
    print("gemm_source_sha256: " + gemm_source_hash())
    print("traffic_bytes: " + json.dumps(traffic))


def short_name(n):
    """Kernel name without namespaces, return type and argument list."""
    n = n.replace("(anonymous namespace)::", "").replace("void ", "").replace("sf::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            return n[:i]
    return n


def kernels(db_path, top):
    """Per (kernel, grid size): launches, total ms, average us, share of the total."""
    import sqlite3
    con = sqlite3.connect(db_path)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    grid = [c for c in ("grid_size", "grid_x") if c in cols]
    q = f"select {name_col}, start, end" + (", " + ", ".join(c for c in ("grid_x", "grid_y", "grid_z") if c in cols)
                                            if "grid_x" in cols else "") + " from kernels"
    agg = {}
    for row in con.execute(q):
        key = (short_name(row[0]), tuple(row[3:]))
        n, t = agg.get(key, (0, 0.0))
        agg[key] = (n + 1, t + (row[2] - row[1]) / 1e6)
    total = sum(t for _, t in agg.values())
    print("| launches | total ms | avg us | % | kernel | grid |")
    print("|---:|---:|---:|---:|:---|:---|")
    for (name, g), (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:top]:
        print(f"| {n} | {t:.3f} | {1000 * t / n:.2f} | {100 * t / total:.2f} | `{name}` | {'x'.join(map(str, g))} |")
    print(f"\ntotal kernel time {total:.3f} ms over {sum(n for n, _ in agg.values())} launches")


def gemm_runs(db_path, workload, min_run=20):
    """The per-role GEMM timing loops of bench.py in a kernel trace: maximal
    runs of >= min_run consecutive launches of one (GEMM kernel, grid),
    split-K reductions in between counted with the GEMM they finish; the last
    12 such runs are the 12 roles in bench.py's order."""
    import sqlite3
    con = sqlite3.connect(db_path)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    rows = con.execute(f"select {name_col}, start, end, grid_x, grid_y from kernels order by start").fetchall()
    runs, cur = [], None
    for name, t0, t1, gx, gy in rows:
        sn = short_name(name)
        if "splitk_reduce" in sn:
            if cur is not None:
                cur["reduce"].append((t1 - t0) / 1e3)
            continue
        key = (sn, gx, gy)
        if cur is not None and cur["key"] == key:
            cur["gemm"].append((t1 - t0) / 1e3)
        else:
            if cur is not None and len(cur["gemm"]) >= min_run:
                runs.append(cur)
            cur = {"key": key, "gemm": [(t1 - t0) / 1e3], "reduce": []}
    if cur is not None and len(cur["gemm"]) >= min_run:
        runs.append(cur)
    roles = _gemms(workload)
    runs = runs[-len(roles):]
    print("| role | kernel | grid | launches | GEMM avg us | split-K reduce avg us | per sf_gemm call us |")
    print("|---|---|---|---:|---:|---:|---:|")
    for (name, lay, M, N, K), r in zip(roles, runs):
        g = sum(r["gemm"]) / len(r["gemm"])
        red = sum(r["reduce"]) / len(r["reduce"]) if r["reduce"] else 0.0
        k, gx, gy = r["key"]
        print(f"| {name} | `{k}` | {gx}x{gy} | {len(r['gemm'])} | {g:.2f} | {red:.2f} | {g + red:.2f} |")


HBM_PEAK = 8.0e12


def rowops(db_path, workload):
    """Achieved HBM bandwidth of the row kernels (see the module docstring)."""
    import sqlite3
    import statistics
    sys.path.insert(0, os.path.dirname(HERE))
    import seeded_inputs as si
    w = si.WORKLOADS[workload]
    e = 4 if w.dtype == "f32" else 2
    T, H, V = w.tokens, w.hidden, w.vocab
    nq = w.n_heads * w.head_dim
    R = min(T, 2048)  # head chunk rows bench.py uses
    con = sqlite3.connect(db_path)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    rows = con.execute(f"select {name_col}, start, end, grid_x from kernels").fetchall()
    # name fragment, launch filter (on its duration in us), algorithmic bytes per launch, what is counted
    spec = [
        ("rmsnorm_fwd_kernel", None, 2 * T * H * e + T * 4 + H * e, "x in, y out, r out"),
        ("rmsnorm_bwd_kernel", None, 4 * T * H * e + T * 4 + H * e, "dy, x, residual in; dx out"),
        # wide rows (a block per row, the row in registers)
        ("rmsnorm_fwd_rows_kernel", None, 2 * T * H * e + T * 4 + H * e, "x in, y out, r out"),
        ("rmsnorm_bwd_rows_kernel", None, 4 * T * H * e + T * 4 + H * e, "dy, x, residual in; dx out"),
        ("gain_partial_kernel", None, 2 * T * H * e + T * 4 + 512 * H * 4, "dy, x in; 512 partial rows out"),
        # fused RMSNorm backward + gain partial sums (hidden <= 2048): 512 row chunks
        ("rmsnorm_bwd_gain_kernel", None, 4 * T * H * e + T * 4 + H * e + 512 * H * 4,
         "dy, x, residual in; dx, 512 partial rows out"),
        ("gain_reduce_kernel", None, 512 * H * 4 + H * 4, "512 partial rows in; gain gradient out"),
        ("attn_dot_kernel", None, 2 * T * nq * e + T * w.n_heads * 4, "dA, O in; row sums out"),
        ("ce_rows_reg_kernel", None, R * V * (4 + e) + R * 8, "fp32 logits in, dlogits out"),
        ("ce_rows_kernel", None, R * V * (4 + e) + R * 8, "fp32 logits in (twice), dlogits out"),
        ("embed_fwd_kernel", None, 2 * T * H * e + T * 4, "rows gathered, x0 out"),
        # the [V, H] tensors' updates (the [H] final gain's take a few us)
        ("adam_device_kernel", lambda us: us > 20.0, V * H * (7 * 4 + e), "g, p, m, v in; p, m, v, bf16 out ([V, H])"),
    ]
    print("| kernel | launches | median us | algorithmic bytes per launch | counted | GB/s | of 8 TB/s |")
    print("|---|---:|---:|---:|---|---:|---:|")
    for frag, gfilter, nbytes, what in spec:
        d = [(t1 - t0) / 1e3 for n, t0, t1, gx in rows
             if frag in short_name(n) and (gfilter is None or gfilter((t1 - t0) / 1e3))
             and not (frag == "ce_rows_kernel" and "ce_rows_reg_kernel" in short_name(n))]
        if not d or nbytes <= 0:
            continue
        us = statistics.median(d)
        gbs = nbytes / (us * 1e-6) / 1e9
        print(f"| `{frag}` | {len(d)} | {us:.1f} | {nbytes / 1e6:.1f} MB | {what} | {gbs:.0f} | "
              f"{100 * gbs * 1e9 / HBM_PEAK:.0f} % |")


def head_study(hidden, vocab, batch, seq, chunks, reps=5):
    """Chunk-size sweep of the fused head (final RMSNorm, logits, cross
    entropy, dx, dW_lm) on synthetic inputs: x ~ N(0, 1), W_lm ~ N(0, 0.02^2),
    g_f = 1, ids ~ U[0, vocab).  chunks: "R" (one dW_lm product per chunk of
    R rows) or "R/D" (dlogits of D rows kept, one dW_lm product per D rows)."""
    import statistics

    import torch

    sys.path.insert(0, os.path.dirname(HERE))
    import seeded_inputs as si
    from layer_sliding_offloaded_amd import runtime as rt
    from layer_sliding_offloaded_amd import sf
    sf.load()
    w = si.WORKLOADS["stack4-h1024-bf16"].with_(hidden=hidden, n_heads=hidden // 128, n_kv_heads=hidden // 128,
                                                head_dim=128, vocab=vocab, batch=batch, seq=seq)
    T = batch * seq
    gen = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(T, hidden, generator=gen, device="cuda").to(torch.bfloat16)
    wlm = (torch.randn(vocab, hidden, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    gf = torch.ones(hidden, device="cuda").to(torch.bfloat16)
    ids = torch.randint(0, vocab, (T,), generator=gen, device="cuda", dtype=torch.int32)
    loss = torch.empty(1, device="cuda")
    dx = torch.empty_like(x)
    dgf = torch.empty(hidden, device="cuda")
    dwlm = torch.empty(vocab, hidden, device="cuda")
    fixed = sum(t.numel() * t.element_size() for t in (x, wlm, gf, ids, loss, dx, dgf, dwlm))
    s = torch.cuda.current_stream()
    flops = 6.0 * T * vocab * hidden
    rows = []
    for spec in chunks:
        R, D = (int(v) for v in spec.split("/")) if "/" in str(spec) else (int(spec), 0)
        shape = rt.shape_from(w)
        L = sf.sf_layer_layout_ex(shape, R, D)
        full = rt.device_bytes(L.workspace_bytes + L.head_workspace_bytes)
        ctx = sf.sf_ctx_create_ex(shape, R, D, full.data_ptr(), full.numel())

        def call():
            sf.sf_head_fwd_bwd(ctx, gf.data_ptr(), wlm.data_ptr(), x.data_ptr(), ids.data_ptr(), loss.data_ptr(),
                               dx.data_ptr(), dgf.data_ptr(), dwlm.data_ptr(), s.cuda_stream)

        for _ in range(2):
            call()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            call()
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = statistics.median(times)
        Dn = min(T, -(-max(D, R) // R) * R)
        rows.append((R, Dn, L.head_workspace_bytes, ms, loss.item()))
        print(f"[head-study] rows {R} dW rows {Dn}: workspace {L.head_workspace_bytes / 2**20:.1f} MiB, {ms:.3f} ms",
              file=sys.stderr, flush=True)
        sf.sf_ctx_destroy(ctx)
        del full
        torch.cuda.synchronize()
    base_ws = max(r[2] for r in rows)
    print(f"Head shape: T = {batch} x {seq} = {T} tokens, hidden {hidden}, vocab {vocab} (bf16, fp32 dW_lm); "
          f"fixed head buffers (x, dx, W_lm, dW_lm, g_f, dg_f, ids, loss): {fixed / 2**30:.3f} GiB.\n")
    print("| chunk rows | dW_lm rows | head workspace (logits fp32 + dlogits bf16 + norm) | vs all rows at once | "
          "head total (workspace + fixed) | vs all rows at once | ms per call | TFLOP/s | loss |")
    print("|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for R, Dn, wsb, ms, lv in rows:
        print(f"| {R} | {Dn} | {wsb / 2**30:.3f} GiB | {100.0 * (1 - wsb / base_ws):.1f} % less | "
              f"{(wsb + fixed) / 2**30:.3f} GiB | {100.0 * (1 - (wsb + fixed) / (base_ws + fixed)):.1f} % less | "
              f"{ms:.3f} | {flops / (ms * 1e-3) / 1e12:.0f} | {lv:.5f} |")


def _union(iv):
    iv = sorted(iv)
    out = []
    for a, b in iv:
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def timeline(path, gap_ms, bucket_ms):
    rows = [(r["kind"], float(r["start_ms"]), float(r["end_ms"]), float(r["info"]))
            for r in csv.DictReader(open(path))]
    kinds = sorted({k for k, _, _, _ in rows})
    t0 = min(a for _, a, _, _ in rows)
    t1 = max(b for _, _, b, _ in rows)
    merged = {k: _union([(a, b) for kk, a, b, _ in rows if kk == k]) for k in kinds}

    def busy(k, lo, hi):
        return sum(max(0.0, min(b, hi) - max(a, lo)) for a, b in merged.get(k, []))

    print(f"window {t1 - t0:.1f} ms, {len(rows)} intervals")
    print()
    print("| kind | busy ms | share of the window | bytes |")
    print("|---|---:|---:|---:|")
    for k in kinds:
        by = sum(x for kk, _, _, x in rows if kk == k and kk in ("h2d", "d2h"))
        print(f"| {k} | {busy(k, t0, t1):.1f} | {100.0 * busy(k, t0, t1) / (t1 - t0):.1f} % | "
              f"{by / 1e9:.2f} GB |" if by else f"| {k} | {busy(k, t0, t1):.1f} | "
              f"{100.0 * busy(k, t0, t1) / (t1 - t0):.1f} % | |")
    d2h = merged.get("d2h", [])
    gaps = [(d2h[i][1], d2h[i + 1][0]) for i in range(len(d2h) - 1) if d2h[i + 1][0] - d2h[i][1] > gap_ms]
    print()
    print(f"Gaps of more than {gap_ms:g} ms without a D2H copy:")
    print()
    print("| from ms | to ms | length ms | H2D busy ms | compute busy ms |")
    print("|---:|---:|---:|---:|---:|")
    for a, b in gaps:
        print(f"| {a - t0:.1f} | {b - t0:.1f} | {b - a:.1f} | {busy('h2d', a, b):.1f} | {busy('compute', a, b):.1f} |")
    print()
    print(f"Busy share per {bucket_ms:g} ms:")
    print()
    print("| ms | " + " | ".join(kinds) + " |")
    print("|---:|" + "---:|" * len(kinds))
    lo = t0
    while lo < t1:
        hi = lo + bucket_ms
        print(f"| {lo - t0:.0f} | " + " | ".join(f"{100.0 * busy(k, lo, hi) / bucket_ms:.0f} %" for k in kinds) + " |")
        lo = hi


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["probe", "summarize", "kernels", "gemm-runs", "rowops", "head-study",
                                     "layer-probe", "mfma", "timeline", "vendor", "vendor-counters"])
    ap.add_argument("files", nargs="*")
    ap.add_argument("--workload", default="stack4-h1024-bf16")
    ap.add_argument("--top", type=int, default=30)
    ap.add_argument("--hidden", type=int, default=4096)
    ap.add_argument("--vocab", type=int, default=128256)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--seq", type=int, default=2048)
    ap.add_argument("--chunks", default="8192,4096,2048,1024,512,256")
    ap.add_argument("--gap", type=float, default=20.0)
    ap.add_argument("--bucket", type=float, default=50.0)
    ap.add_argument("--gemms", default="")
    ap.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    if a.mode == "probe":
        probe(a.workload)
    elif a.mode == "layer-probe":
        layer_probe(a.workload)
    elif a.mode == "mfma":
        mfma(a.files[0], a.workload)
    elif a.mode == "summarize":
        summarize(a.files[0], a.files[1], a.workload)
    elif a.mode == "gemm-runs":
        gemm_runs(a.files[0], a.workload)
    elif a.mode == "rowops":
        rowops(a.files[0], a.workload)
    elif a.mode == "head-study":
        head_study(a.hidden, a.vocab, a.batch, a.seq, a.chunks.split(","))
    elif a.mode == "vendor":
        vendor(a.workload, a.gemms, a.reps)
    elif a.mode == "vendor-counters":
        vendor_counters(a.files, a.workload, a.gemms, a.reps)
    elif a.mode == "timeline":
        timeline(a.files[0], a.gap, a.bucket)
    else:
        kernels(a.files[0], a.top)


if __name__ == "__main__":
    main()
