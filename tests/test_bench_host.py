"""Host logic of bench.py (no GPU): the algorithmic byte counts it reports,
the one-GPU refusal, and the rule that a committed traffic profile counts
only for the kernel sources it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_one_ling_layer():
    # one routed expert: gate_up codes 2*768*2560/2 + scales 2*768*80*2, down
    # codes 2560*768/2 + scales 2560*24*2
    assert bench.EXPERT_GU_BYTES == 1_966_080 + 245_760
    assert bench.EXPERT_DN_BYTES == 983_040 + 122_880
    assert bench.EXPERT_BYTES == 3_317_760
    assert bench.SHARED_GU_BYTES + bench.SHARED_DN_BYTES == 11_796_480
    assert bench.ROUTER_BYTES == 5_242_880
    # decode: 8 experts + shared + router + x in and out
    assert bench.step_bytes(8, 1) == 43_591_680
    # verify: distinct experts counted once, tokens' rows per token
    assert bench.step_bytes(31, 4) - bench.step_bytes(31, 1) == 3 * 2 * 2560 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_profile_counts_only_for_its_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("some_workload") is None  # no profile
    digest = "0" * 64

    def write(d):
        (prof / "some_workload_traffic.txt").write_text(
            f"header line\nkernel: k\nhbm_bytes_per_launch: 123456\nsources_sha256: {d}\n")

    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: digest)
    write(digest)
    assert bench.measured_traffic("some_workload") == 123456
    write("f" * 64)
    assert bench.measured_traffic("some_workload") is None


def test_sources_digest_covers_every_kernel_source():
    d1 = bench.kernel_sources_digest()
    assert len(d1) == 64 and d1 == bench.kernel_sources_digest()
    csrc = os.path.join(ROOT, "w4a16_grouped_quantized_amd", "csrc")
    names = [n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp"))]
    assert {"layer.hip", "experts.hip", "prefill.hip", "route_dev.hpp", "common.hpp"} <= set(names)
    # only the read-rate probe, which no layer kernel includes, is left out
    assert set(bench.DIGEST_EXCLUDED) == {"probe.hip"}
    for n in names:
        if n != "probe.hip":
            assert '#include "probe' not in open(os.path.join(csrc, n)).read()


def test_source_digest_ignores_comments_not_code():
    src = 'int a = 1; // note\n/* block\n comment */ int b = 2;\n\n  const char* s = "//x/*y*/";  \nchar q = \'"\';\n'
    got = bench.source_code_only(src)
    assert got == 'int a = 1;\n  int b = 2;\n  const char* s = "//x/*y*/";\nchar q = \'"\';'
    assert bench.source_code_only(src.replace("note", "other note")) == got
    assert bench.source_code_only(src.replace("b = 2", "b = 3")) != got

