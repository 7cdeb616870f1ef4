"""GPU parity of the NF4 codec kernels: quantise bytes and dequantise bits
must equal the oracle's exactly (integer/byte work is bit-exact)."""

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, bits_of, code_tensors, ref_bits, to_dev, upload

pytestmark = pytest.mark.gpu

# ragged sizes: element counts not multiple of 64 / 8, nested groups partial
PLAIN_SHAPES = [(128, 256), (3, 66), (1, 2), (77, 64), (5, 190), (1024, 4096)]
NESTED_SHAPES = [(128, 256), (7, 640), (300, 1024), (33, 130), (4096, 4096)]


def _w(N, K, seed):
    return WL.weight_f32(N, K, WL.W_TINY, 100 + seed)


def _quant_gpu(w, nested, bf16=False):
    code, ncode = code_tensors(nested)
    wt = torch.from_numpy(w).to(DEV)
    if bf16:
        wt = wt.to(torch.bfloat16)
    return api.nf4_quantize(wt, code, ncode)


def _check_quant(q, ref, nested):
    assert np.array_equal(q.packed.cpu().numpy(), ref["packed"]), "packed bytes differ"
    if nested:
        assert np.array_equal(q.absmax.cpu().numpy(), ref["absmax"]), "nested u8 absmax differs"
        assert np.array_equal(q.nested_absmax.cpu().numpy(), ref["nested_absmax"]), "s2 differs"
        assert q.nested_offset.cpu().numpy()[0] == ref["nested_offset"], "offset differs"
    else:
        assert np.array_equal(q.absmax.cpu().numpy(), ref["absmax"]), "absmax differs"


@pytest.mark.parametrize("N,K", PLAIN_SHAPES)
def test_quantize_plain(N, K):
    w = _w(N, K, N + K)
    w.reshape(-1)[::17] = 0.0
    _check_quant(_quant_gpu(w, False), O.quantize_nf4(w), False)


@pytest.mark.parametrize("N,K", NESTED_SHAPES)
def test_quantize_nested(N, K):
    w = _w(N, K, 7 * N + K)
    _check_quant(_quant_gpu(w, True), O.quantize_nf4(w, nested=True), True)


def test_quantize_bf16_input():
    w = _w(256, 512, 3)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    widened = wb.float().numpy()                       # exact widening, done by torch
    for nested in (False, True):
        _check_quant(_quant_gpu(w, nested, bf16=True), O.quantize_nf4(widened, nested=nested), nested)


def test_quantize_zero_blocks_and_tie_values():
    code = O.nf4_code()
    mids = O.midpoints(code)
    w = np.zeros((4, 64), np.float32)
    w[1, 0] = 1.0
    w[1, 1:16] = mids                                  # exact midpoints -> lower code
    w[2] = (np.tile(code, 4) * np.float32(2.0)).astype(np.float32)
    w[3, ::2] = -0.5
    for nested in (False, True):
        _check_quant(_quant_gpu(w, nested), O.quantize_nf4(w, nested=nested), nested)


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("N,K", [(128, 256), (3, 66), (300, 1024), (1, 2)])
def test_dequantize_bit_exact(N, K, nested):
    w = _w(N, K, 11 * N + K)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    got = api.nf4_dequantize(wq, torch.bfloat16)
    assert np.array_equal(bits_of(got), ref_bits(ref, (N, K))), "bf16 dequant bits differ"
    got32 = api.nf4_dequantize(wq, torch.float32).cpu().numpy()
    want32 = O.dequantize_nf4_f32(ref["packed"], ref["absmax"], ref["nested_absmax"],
                                  ref["nested_offset"]).reshape(N, K)
    assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32)), "fp32 dequant differs"


@pytest.mark.parametrize("proj", ["k", "gate", "down"])
def test_llama_layer_weights_codec(proj):
    """Full-size Llama-3.1-8B projection weights, nested: quantise bytes and
    dequantise bits equal the oracle's."""
    p = {q.name: q for q in WL.LLAMA_8B}[proj]
    w = WL.weight_f32(p.N, p.K, WL.W_LLAMA, 0, WL.LLAMA_8B.index(p))
    ref = O.quantize_nf4(w, nested=True)
    q = _quant_gpu(w, True)
    _check_quant(q, ref, True)
    got = api.nf4_dequantize(q, torch.bfloat16)
    assert np.array_equal(bits_of(got), ref_bits(ref, (p.N, p.K)))


def test_qwen_gate_codec():
    p = WL.QWEN_32B[4]
    w = WL.weight_f32(p.N, p.K, WL.W_QWEN, 0, 4)
    ref = O.quantize_nf4(w, nested=True)
    q = _quant_gpu(w, True)
    _check_quant(q, ref, True)
