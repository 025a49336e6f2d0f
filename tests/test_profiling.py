"""Host logic of the profile summaries that bench.py reads: a traffic figure
is used only while the kernel code it was measured on is unchanged."""
import os
import re

from fp4_quantized_moe_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_hash_ignores_comments_only():
    a = "int f(int x) { // doubled\n  return 2 * x; /* no overflow */ }\n"
    b = "int f(int x) {\n\n  return 2 * x;  }  // changed comment\n"
    c = "int f(int x) { return 3 * x; }"
    assert P._code_only(a) == P._code_only(b)
    assert P._code_only(a) != P._code_only(c)


def test_read_traffic_checks_source_hash(tmp_path):
    src = os.path.join(ROOT, "profiles", "k_gemm_dma_expert_gemm_k50_traffic.txt")
    text = open(src).read()
    good = tmp_path / "good.txt"
    good.write_text(re.sub(r"source_sha256: \w+", "source_sha256: " + P.sources_sha256("k_gemm"), text))
    val, fields = P.read_traffic(str(good))
    assert val == float(fields["traffic_bytes_per_launch"]) and val > 0
    stale = tmp_path / "stale.txt"
    stale.write_text(re.sub(r"source_sha256: \w+", "source_sha256: " + "0" * 64, text))
    assert P.read_traffic(str(stale))[0] is None
    assert P.read_traffic(str(tmp_path / "missing.txt"))[0] is None
