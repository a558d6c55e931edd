"""Host logic of bench.py's roofline record (no GPU): the kernel source hash
that ties a committed counter profile to the code it was taken on, and the
traffic lookup that uses it."""
import os
import re

import bench


def test_code_text_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ int y = x + 2;\n"
    b = "int x = 1;\n\n   int y = x + 2;   // two\n"
    assert bench.code_text(a) == bench.code_text(b) == "int x = 1; int y = x + 2;"
    # a change to the code itself changes the text
    assert bench.code_text(a) != bench.code_text(a.replace("x + 2", "x + 3"))


def test_traffic_lookup_follows_the_code(tmp_path, monkeypatch):
    """A counter summary is used while the hash it records matches the
    kernel's code; an edit to comments keeps it, an edit to code retires it."""
    csrc = tmp_path / "paged_kv_cache_134_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": ["k.hip"]})
    src = csrc / "k.hip"
    src.write_text("__global__ void k() { int a = 1; }  // first\n")
    (tmp_path / "profiles" / "k_w_traffic.txt").write_text(
        f"kernel_source_sha: {bench.source_sha('k')}\nhbm_bytes_per_launch: 1234\n")
    assert bench.traffic_from_profile("w", "k") == 1234.0
    src.write_text("/* reworded */ __global__ void k() {\n  int a = 1;\n}\n")
    assert bench.traffic_from_profile("w", "k") == 1234.0
    src.write_text("__global__ void k() { int a = 2; }\n")
    assert bench.traffic_from_profile("w", "k") is None
    assert bench.traffic_from_profile("missing", "k") is None
