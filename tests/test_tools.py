"""Host logic of the measurement tools: kernel-name shortening and the rule
that a stored HBM-traffic figure is used only for the GEMM source it was
measured on."""

import json

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

