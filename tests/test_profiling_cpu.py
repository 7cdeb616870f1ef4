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


def test_counter_summary_scales_by_the_copy(tmp_path):
    """Fused dispatches summed per operation; FETCH_SIZE scaled by the factor
    that maps the calibration copy's count onto its known size; other
    kernels ignored."""
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for d in range(4):                                  # two ops of two dispatches each
        rows.append(f'{d},"void nf4::k_gemv_ln<4, 2, true, 16>(GemvArgs)",FETCH_SIZE,100')
        rows.append(f'{d},"void nf4::k_gemv_ln<4, 2, true, 16>(GemvArgs)",SQ_INSTS_VALU,7')
    rows.append("9,__amd_rocclr_copyBuffer,FETCH_SIZE,512")       # 1 MiB copy counted as 512 KiB
    rows.append("9,__amd_rocclr_copyBuffer,SQ_INSTS_VALU,3")
    rows.append("10,void other_kernel(),FETCH_SIZE,99999")
    rows.append("10,void other_kernel(),SQ_INSTS_VALU,99999")
    path = tmp_path / "pmc.csv"
    path.write_text("\n".join(rows) + "\n")
    fig = P.counter_figures(str(path), 1 << 20, 2, 300 * 1024.0)
    assert fig["fused_dispatches"] == 4
    assert fig["per_op"]["FETCH_SIZE"] == 200.0 and fig["per_op"]["SQ_INSTS_VALU"] == 14.0
    assert fig["FETCH_SIZE_factor"] == 2.0
    assert fig["FETCH_SIZE_bytes_per_op"] == 400 * 1024
    assert abs(fig["FETCH_SIZE_over_algorithmic"] - 4 / 3) < 1e-3
