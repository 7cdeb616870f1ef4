"""Host logic of the profile summaries: the kernel-source hash that ties a
counter figure to the code it was measured on ignores comments and layout but
not code, and the committed traffic summary parses."""

import os

from nf4_bit_weight_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_strips_comments_not_literals():
    src = 'int a = 1; // c\n/* block\n comment */ char s[] = "// kept"; char q = \'/\';\n\n  int b;'
    assert P._code_only(src) == 'int a = 1; char s[] = "// kept"; char q = \'/\'; int b;'
    assert P._code_only("x = y; // note") == P._code_only("x  =  y;\n/* other note */")
    assert P._code_only("x = y;") != P._code_only("x = z;")


def test_traffic_summary_parses():
    path = os.path.join(ROOT, "profiles", "traffic_fused_gemm_bwd_down_m512.md")
    text = open(path).read()
    assert "FETCH_SIZE" in text and "WRITE_SIZE" in text and "kernel_source_sha256" in text
