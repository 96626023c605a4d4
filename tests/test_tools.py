"""Host logic of the measurement tools: kernel-name shortening, the rule
that a stored HBM-traffic figure is used only for the GEMM source it was
measured on, the engine-timeline summary and the pairing of counter rows
in the comparison with the vendor library."""

import json

import pytest

import bench
from layer_sliding_offloaded_amd import prof


def test_short_name_drops_namespaces_and_arguments():
    n = ("void sf::(anonymous namespace)::gemm_pp_kernel<256, 256, 128, 64, 32, (sf::GemmLayout)0, (sf::Epi)0, 4>"
         "(sf::GemmArgs, int, int, int, int)")
    assert prof.short_name(n) == "gemm_pp_kernel<256, 256, 128, 64, 32, (GemmLayout)0, (Epi)0, 4>"
    assert prof.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_stored_traffic_requires_matching_source(tmp_path, monkeypatch):
    prof_dir = tmp_path / "profiles"
    prof_dir.mkdir()
    table = {"gu_dw": 123456}
    path = prof_dir / "gemm_traffic_w.md"
    path.write_text("gemm_source_sha256: " + prof.gemm_source_hash() + "\ntraffic_bytes: " + json.dumps(table) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("w", "gu_dw") == 123456
    assert bench.stored_traffic("w", "qkv_fwd") is None
    assert bench.stored_traffic("other", "gu_dw") is None
    path.write_text("gemm_source_sha256: 0000\ntraffic_bytes: " + json.dumps(table) + "\n")
    assert bench.stored_traffic("w", "gu_dw") is None



def test_timeline_busy_times_and_d2h_gaps(tmp_path, capsys):
    """Overlapping intervals of one kind count once; a D2H gap is reported
    with the H2D and compute time inside it."""
    rows = [("compute", 0, 10), ("compute", 5, 20), ("d2h", 0, 30), ("d2h", 100, 150), ("h2d", 40, 90),
            ("compute", 60, 70)]
    path = tmp_path / "t.csv"
    path.write_text("kind,start_ms,end_ms,info\n" + "".join(f"{k},{a},{b},1000000000\n" for k, a, b in rows))
    prof.timeline(str(path), 20.0, 50.0)
    out = capsys.readouterr().out
    assert "window 150.0 ms" in out
    assert "| compute | 30.0 | 20.0 % | |" in out
    assert "| d2h | 80.0 | 53.3 % | 2.00 GB |" in out
    assert "| 30.0 | 100.0 | 70.0 | 50.0 | 10.0 |" in out


def test_vendor_counters_pairs_launches_by_order(tmp_path, capsys):
    """Per GEMM the CSV holds this library's launches, then the library's
    (two warm-ups + reps each), among unrelated kernels; each side's counters
    are averaged over its timed launches only, and a launch sequence that does
    not have that shape is refused."""
    reps = 2
    rows, d = [], 0
    for g in ("o_fwd", "o_dx"):
        for kind, base in (("_ZN2sf12gemm_pp_kernel", 100.0), ("Cijk_Ailk_Bljk_MT256x256x64_SK3", 10.0)):
            for i in range(2 + reps):
                d += 1
                rows.append((d, "randn_kernel", "X", 1.0))
                d += 1
                v = base * (1 if g == "o_fwd" else 2) + (1000.0 if i < 2 else i)
                rows.append((d, kind, "TCC_MISS_sum", v))
    path = tmp_path / "c.csv"
    path.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n" +
                    "".join(f"{a},{b},{c},{v},0,1000\n" for a, b, c, v in rows))
    prof.vendor_counters([str(path)], "slice123b-gqa-bf16", "o_fwd,o_dx", reps)
    out = capsys.readouterr().out.splitlines()
    got = {(l.split("|")[1].strip(), "Cijk" in l or "MT256" in l): float(l.split("|")[4]) for l in out[2:]}
    # timed launches carry base * g + 2 and + 3: mean base * g + 2.5
    assert got == {("o_fwd", False): 102.5, ("o_fwd", True): 12.5, ("o_dx", False): 202.5, ("o_dx", True): 22.5}
    with pytest.raises(SystemExit):
        prof.vendor_counters([str(path)], "slice123b-gqa-bf16", "o_fwd,o_dx", reps + 1)


def test_layer_gemms_cover_the_projection_flops():
    """The 12 GEMMs timed one by one are exactly the dense part of a layer's
    forward + backward: forward, dX and dW each multiply the T tokens by every
    projection weight once (2 T P flops apiece), so their sum is 6 T P_lin --
    the non-attention term of layer_flops.  Checked on shapes with GQA and
    with n_heads * head_dim != hidden, where a transposed or dropped GEMM
    changes the sum."""
    import seeded_inputs as si
    for name, w in si.WORKLOADS.items():
        gemm = sum(2.0 * M * N * K for _, _, M, N, K in prof.layer_gemms(w))
        attn = 6.0 * w.batch * w.n_heads * w.seq * w.seq * w.head_dim
        assert gemm + attn == prof.layer_flops(w), name
    w = si.WORKLOADS["stack4-h1024-bf16"].with_(n_heads=6, n_kv_heads=2, head_dim=96, hidden=512, ffn=768)
    T, H = w.tokens, w.hidden
    p_lin = H * 96 * (6 + 2 + 2) + 6 * 96 * H + 3 * 768 * H
    gemm = sum(2.0 * M * N * K for _, _, M, N, K in prof.layer_gemms(w))
    assert gemm == 6.0 * T * p_lin
    # every GEMM's reduction length is one of the layer's own widths
    for _, lay, M, N, K in prof.layer_gemms(w):
        assert K in (H, 6 * 96, 2 * 768, 768, (6 + 4) * 96, T)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
