"""GPU parity of the 8-bit blockwise variants (bitsandbytes fork PR
"Experts trainability ... ExpertsNbit", "Commit 1" quant_type table: int8 and
fp8 e4m3 blockwise, one byte per weight) against the oracle:

* codec: quantised bytes and statistics byte-exact, dequantised weights
  bit-exact in bf16 and fp32, for the int8 and the e4m3 table, plain and
  nested, including odd element counts, all-zero blocks and exact midpoints;
* fused matmuls (forward and input gradient, 128-row tiles and the 32-row
  small-M tiles with a split contraction): tolerance against the oracle on
  ragged shapes, bit-exact identity probes in both orientations, bitwise
  repeats, the path counters of the 8-bit kernels;
* grouped experts, the autograd wrapper, and one Llama-3.1-8B-shaped
  projection at M = 512 checked on sampled columns.
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

TABLES = {"int8": WL.int8_code_np, "fp8": WL.fp8_e4m3_code_np}


def _ref(w, table, nested):
    return O.quantize_blockwise8(w.reshape(-1), TABLES[table](), nested=nested)


def _upload(ref, N, K, table, nested):
    code = to_dev(TABLES[table]())
    if nested:
        return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]), to_dev(ref["nested_absmax"]),
                         to_dev(np.array([ref["nested_offset"]], np.float32)), code,
                         to_dev(WL.nested_code_np()), N, K, 8)
    return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]), None, None, code, None, N, K, 8)


def _bits(ref, table, shape):
    return O.dequantize_blockwise8_bf16_bits(ref["packed"], ref["absmax"], ref["nested_absmax"],
                                             ref["nested_offset"], code=TABLES[table]()).reshape(shape)


def _weight(N, K, table, nested, seed):
    w = WL.weight_f32(N, K, WL.W_TINY, 3000 + seed)
    ref = _ref(w, table, nested)
    return _upload(ref, N, K, table, nested), _bits(ref, table, (N, K))


@pytest.mark.parametrize("table", ["int8", "fp8"])
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("N,K", [(128, 256), (37, 129), (512, 520)])
def test_codec_8bit_bit_exact(N, K, nested, table):
    w = WL.weight_f32(N, K, WL.W_TINY, 3100 + N + K)
    w[3, :] = 0.0                                        # zero blocks
    code = TABLES[table]()
    mids = O.midpoints(code)
    w[5, :8] = mids[100:108]                             # t lands exactly on midpoints:
    w[5, 8] = 1.0                                        # the block's absmax is 1 (ties go low)
    ref = _ref(w, table, nested)
    got = api.nf4_quantize_8bit(to_dev(w), to_dev(code), to_dev(WL.nested_code_np()) if nested else None)
    torch.cuda.synchronize()
    assert np.array_equal(got.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(got.absmax.cpu().numpy().view(np.uint8 if nested else np.float32), ref["absmax"])
    if nested:
        assert np.array_equal(got.nested_absmax.cpu().numpy(), ref["nested_absmax"])
        assert got.nested_offset.cpu().numpy()[0] == ref["nested_offset"]
    wb = api.nf4_dequantize(got)
    assert np.array_equal(bits_of(wb).reshape(-1), _bits(ref, table, (-1,)))
    wf = api.nf4_dequantize(got, out_dtype=torch.float32).cpu().numpy().reshape(-1)
    want = O.dequantize_blockwise8_f32(ref["packed"], ref["absmax"], ref["nested_absmax"],
                                       ref["nested_offset"], code=code)
    assert np.array_equal(wf.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("table", ["int8", "fp8"])
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 136, 192), (8, 264, 320), (32, 1024, 2048), (100, 392, 704),
                                   (513, 136, 1088), (256, 512, 1024)])
def test_matmul_8bit_vs_oracle(M, N, K, nested, table):
    wq, wb = _weight(N, K, table, nested, M + N + K)
    x = WL.x_bf16(M, K, WL.W_TINY, 3200 + M)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 3200 + M)
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx2 = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    torch.cuda.synchronize()
    c = api.nf4_path_counts()
    assert c["fwd_8bit"] == 2 and c["bwd_8bit"] == 2
    assert c["fwd_tiled"] == c["fwd_small_m"] == c["bwd_tiled"] == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))
    assert_close(y, O.matmul_fwd(xb, wb), f"y {M}x{N}x{K}", O.matmul_fwd(abs_bits(xb), aw), K)
    assert_close(gx, O.matmul_bwd_input(gyb, wb), f"gx {M}x{N}x{K}", O.matmul_bwd_input(abs_bits(gyb), aw), N)


def _plus_zero(b):
    """bf16 bits with -0 mapped to +0: the e4m3 table decodes a zero weight as
    -0 (its lower index), while the fp32 accumulators start from +0."""
    b = np.asarray(b, dtype=np.uint16)
    return np.where(b == 0x8000, np.uint16(0), b)


@pytest.mark.parametrize("table", ["int8", "fp8"])
@pytest.mark.parametrize("M", [8, 200])
def test_identity_probes_8bit(M, table):
    """Unit rows of x give rows of W_hat^T, unit rows of grad_y rows of W_hat,
    bit for bit (up to the sign of zero), on the small-M and the 128-row
    tiles."""
    N, K = 320, 384
    wq, wb = _weight(N, K, table, True, 7 + M)
    g = np.random.default_rng(M)
    p = g.integers(0, K, size=M)
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[np.arange(M), p] = 1.0
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert np.array_equal(_plus_zero(bits_of(y)), _plus_zero(wb.T[p]))
    q = g.integers(0, N, size=M)
    gy = torch.zeros((M, N), dtype=torch.bfloat16)
    gy[np.arange(M), q] = 1.0
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert np.array_equal(_plus_zero(bits_of(gx)), _plus_zero(wb[q]))


@pytest.mark.parametrize("table", ["int8", "fp8"])
@pytest.mark.parametrize("counts", [(3, 0, 70, 129, 0, 1), (300, 0, 5, 411, 260, 0)])
def test_grouped_8bit(table, counts):
    """Few rows per expert (32-row tiles) and many (128-row tiles), with
    empty experts and ragged row counts."""
    E, N, K = len(counts), 136, 192
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    w = WL.weight_f32(E * N, K, WL.W_OLMOE, 3300)
    ref = _ref(w, table, True)
    wq = _upload(ref, E * N, K, table, True).per_expert(E)
    wb = _bits(ref, table, (E, N, K))
    x = WL.x_bf16(T, K, WL.W_OLMOE, 3301)
    gy = WL.grad_y_bf16(T, N, WL.W_OLMOE, 3302)
    off = torch.from_numpy(offsets).to(DEV)
    y = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
    gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    gx2 = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), "grouped y",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, aw), K)
    assert_close(gx, O.grouped_matmul_bwd_input(gyb, offsets, wb), "grouped gx",
                 O.grouped_matmul_bwd_input(abs_bits(gyb), offsets, aw), N)


def test_autograd_wrapper_8bit():
    from nf4_bit_weight_amd.autograd import nf4_linear
    N, K, M = 256, 512, 64
    wq, wb = _weight(N, K, "int8", True, 11)
    x = WL.x_bf16(M, K, WL.W_TINY, 3400).to(DEV).requires_grad_(True)
    y = nf4_linear(x, wq)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 3401).to(DEV)
    y.backward(gy)
    assert torch.equal(y.view(torch.int16), api.nf4_matmul_fwd(x.detach(), wq).view(torch.int16))
    assert torch.equal(x.grad.view(torch.int16), api.nf4_matmul_bwd_input(gy, wq).view(torch.int16))


@pytest.mark.parametrize("table", ["int8", "fp8"])
def test_llama_q_shape_8bit_sampled(table):
    """Llama-3.1-8B q projection (4096 x 4096) at M = 512, nested, quantised
    on the device (its bytes checked against the oracle), fused forward and
    input gradient checked on 48 sampled columns each."""
    N = K = 4096
    M = 512
    w = WL.weight_f32(N, K, WL.W_LLAMA, 3500)
    ref = _ref(w, table, True)
    code = to_dev(TABLES[table]())
    wq = api.nf4_quantize_8bit(to_dev(w), code, to_dev(WL.nested_code_np()))
    assert np.array_equal(wq.packed.cpu().numpy(), ref["packed"])
    wb = _bits(ref, table, (N, K))
    x = WL.x_bf16(M, K, WL.W_LLAMA, 3501)
    gy = WL.grad_y_bf16(M, N, WL.W_LLAMA, 3502)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    g = np.random.default_rng(5)
    cn = np.sort(g.choice(N, 48, replace=False))
    ck = np.sort(g.choice(K, 48, replace=False))
    xb, gyb = WL.bf16_bits(x), WL.bf16_bits(gy)
    assert_close(y[:, torch.from_numpy(cn).to(DEV)], O.matmul_fwd(xb, wb[cn]), "y sampled",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb[cn])), K)
    assert_close(gx[:, torch.from_numpy(ck).to(DEV)], O.matmul_bwd_input(gyb, wb[:, ck]), "gx sampled",
                 O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb[:, ck])), N)
