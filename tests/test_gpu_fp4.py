"""The fp4 code table through the same kernels (a 16-entry table swap).

The Experts PR ("Commit 1" table) lists nf4 and fp4 on one 4-bit packed
path.  The table is a call argument, so every kernel runs unchanged; these
tests pass the fp4 table to the quantiser, the dequantiser, the tiled and
weight-streaming forwards, the input gradient and the grouped forward, and
check each against the oracle given the same table: bytes and dequantised
bits exactly (including the -0 entry), matmul outputs within the GEMM
tolerance.
"""

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from nf4_bit_weight_amd.api import NF4Weight
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, bits_of, to_dev

pytestmark = pytest.mark.gpu

FP4 = WL.fp4_code_np()


def _tables(nested):
    return to_dev(FP4), (to_dev(WL.nested_code_np()) if nested else None)


def _ref(w, nested):
    return O.quantize_nf4(w, code=FP4, nested=nested)


def _ref_bits(ref, shape):
    return O.dequantize_nf4_bf16_bits(ref["packed"], ref["absmax"], ref["nested_absmax"],
                                      ref["nested_offset"], code=FP4).reshape(shape)


def _upload(ref, N, K, nested):
    code, ncode = _tables(nested)
    if nested:
        return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]), to_dev(ref["nested_absmax"]),
                         to_dev(np.array([ref["nested_offset"]], np.float32)), code, ncode, N, K)
    return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]), None, None, code, None, N, K)


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("N,K", [(128, 256), (33, 130), (300, 1024)])
def test_fp4_codec_bit_exact(N, K, nested):
    w = WL.weight_f32(N, K, WL.W_TINY, 500 + N + K)
    w.reshape(-1)[::13] = 0.0                       # exact zeros take the -0 entry
    ref = _ref(w, nested)
    code, ncode = _tables(nested)
    q = api.nf4_quantize(torch.from_numpy(w).to(DEV), code, ncode)
    assert np.array_equal(q.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(q.absmax.cpu().numpy(), ref["absmax"])
    if nested:
        assert np.array_equal(q.nested_absmax.cpu().numpy(), ref["nested_absmax"])
        assert q.nested_offset.cpu().numpy()[0] == ref["nested_offset"]
    want = _ref_bits(ref, (N, K))
    assert np.array_equal(bits_of(api.nf4_dequantize(q)), want)
    assert np.any(want == 0x8000), "the -0 entry must appear as bf16 -0"


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 200, 576), (17, 136, 448), (64, 256, 512), (300, 520, 1088)])
def test_fp4_matmul_vs_oracle(M, N, K, nested):
    w = WL.weight_f32(N, K, WL.W_TINY, 600 + M + N)
    ref = _ref(w, nested)
    wq = _upload(ref, N, K, nested)
    wb = _ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, 600 + M)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 600 + M)
    xb, gb = WL.bf16_bits(x), WL.bf16_bits(gy)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    g = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    torch.cuda.synchronize()
    c = api.nf4_path_counts()
    assert c["fwd_small_m" if M <= 32 else "fwd_tiled"] == 1 and c["bwd_tiled"] == 1
    assert_close(y, O.matmul_fwd(xb, wb), "fp4 fwd", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    assert_close(g, O.matmul_bwd_input(gb, wb), "fp4 bwd", O.matmul_bwd_input(abs_bits(gb), abs_bits(wb)), N)


def test_fp4_grouped_fwd_vs_oracle():
    E, N, K = 4, 64, 256
    w = WL.weight_f32(E * N, K, WL.W_TINY, 700)
    ref = _ref(w, True)
    wq = _upload(ref, E * N, K, True).per_expert(E)
    wb = _ref_bits(ref, (E, N, K))
    offsets = np.array([0, 37, 37, 130, 161], dtype=np.int32)     # one empty expert
    T = int(offsets[-1])
    x = WL.x_bf16(T, K, WL.W_TINY, 701)
    y = api.nf4_grouped_matmul_fwd(x.to(DEV), to_dev(offsets), wq, E)
    xb = WL.bf16_bits(x)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), "fp4 grouped fwd",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, abs_bits(wb)), K)
