"""GPU parity of the grouped (expert) forward and input gradient."""

import os

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, ref_bits, upload

pytestmark = pytest.mark.gpu


def _stack(E, N, K, nested, seed):
    w = WL.weight_f32(E * N, K, WL.W_OLMOE, seed)
    ref = O.quantize_nf4(w, nested=nested)
    return upload(ref, N, K, nested), ref_bits(ref, (E, N, K))


@pytest.mark.parametrize("nested", [False, True])
def test_grouped_ragged_and_empty_experts(nested):
    E, N, K = 6, 136, 192
    counts = np.array([3, 0, 70, 129, 0, 1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    wq, wb = _stack(E, N, K, nested, 5)
    x = WL.x_bf16(T, K, WL.W_OLMOE, 50)
    gy = WL.grad_y_bf16(T, N, WL.W_OLMOE, 50)
    off = torch.from_numpy(offsets).to(DEV)
    y = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
    gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), "grouped y",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, aw), K)
    assert_close(gx, O.grouped_matmul_bwd_input(gyb, offsets, wb), "grouped grad_x",
                 O.grouped_matmul_bwd_input(abs_bits(gyb), offsets, aw), N)


def test_grouped_identity_rows():
    """Each routed row is a unit vector: outputs are exact columns of W_hat_e."""
    E, N, K = 4, 64, 128
    wq, wb = _stack(E, N, K, True, 6)
    counts = np.array([5, 9, 0, 2])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    p = np.random.default_rng(3).integers(0, K, size=T)
    x = torch.zeros((T, K), dtype=torch.bfloat16)
    x[np.arange(T), p] = 1.0
    y = api.nf4_grouped_matmul_fwd(x.to(DEV), torch.from_numpy(offsets).to(DEV), wq, E)
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    exp = np.repeat(np.arange(E), counts)
    want = np.stack([wb[exp[t], :, p[t]] for t in range(T)])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nested", [False, True])
def test_grouped_transposed_identity_rows(nested):
    """Each routed row of grad_y is a unit vector e_j: the input gradient's row
    is row j of W_hat_e, bit for bit (the transposed read of the same packed
    stack)."""
    E, N, K = 5, 72, 192
    wq, wb = _stack(E, N, K, nested, 16)
    counts = np.array([7, 0, 3, 12, 1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    j = np.random.default_rng(4).integers(0, N, size=T)
    gy = torch.zeros((T, N), dtype=torch.bfloat16)
    gy[np.arange(T), j] = 1.0
    off = torch.from_numpy(offsets).to(DEV)
    gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    got = gx.cpu().view(torch.int16).numpy().view(np.uint16)
    exp = np.repeat(np.arange(E), counts)
    want = np.stack([wb[exp[t], j[t], :] for t in range(T)])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_olmoe_experts(proj):
    """OLMoE-1B-7B experts: 512 tokens, top-8 of 64, nested NF4 stacks."""
    E, H, I = WL.OLMOE_E, WL.OLMOE_HIDDEN, WL.OLMOE_INTER
    N, K = (I, H) if proj == "gate" else (H, I)
    _, _, offsets = WL.olmoe_routing()
    T = int(offsets[-1])
    assert T == WL.OLMOE_TOKENS * WL.OLMOE_TOPK
    wq, wb = _stack(E, N, K, True, 10 + (proj == "down"))
    x = WL.x_bf16(T, K, WL.W_OLMOE, 60)
    gy = WL.grad_y_bf16(T, N, WL.W_OLMOE, 61)
    off = torch.from_numpy(offsets).to(DEV)
    y = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
    gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), f"olmoe {proj} y",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, aw), K)
    assert_close(gx, O.grouped_matmul_bwd_input(gyb, offsets, wb), f"olmoe {proj} gx",
                 O.grouped_matmul_bwd_input(abs_bits(gyb), offsets, aw), N)
    # bitwise run-to-run repeat of both directions, the second run after an
    # unrelated launch of the other direction on other inputs
    api.nf4_grouped_matmul_fwd(torch.flip(x, [0]).to(DEV), off, wq, E)
    gx2 = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
    api.nf4_grouped_matmul_bwd_input(torch.flip(gy, [0]).to(DEV), off, wq, E)
    y2 = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))


@pytest.mark.parametrize("bm,bn,consumers", [(64, 256, 1), (64, 128, 1), (128, 256, 1), (128, 256, 2),
                                             (128, 128, 1), (256, 256, 4), (256, 256, 0), (256, 128, 0),
                                             (128, 128, 5), (64, 128, 5), (32, 128, 5),
                                             (128, 128, 6), (64, 128, 6), (128, 256, 6)])
def test_grouped_tiles(bm, bn, consumers):
    """Every tile the grouped products can be given through NF4_BM / NF4_BN /
    NF4_CONSUMERS, on ragged experts (empty ones, one spanning two 128-row
    tiles): 256 x 256 is the ping-pong kernel in both directions with
    consumers 4 and the register-operand forward with 0, 256 x 128 the
    4-wave register-operand forward, consumers 5 / 6 the register-staged tile
    kernel with 4 / 8 waves."""
    E, N, K = 6, 136, 192
    counts = np.array([3, 0, 70, 129, 0, 1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    wq, wb = _stack(E, N, K, True, 9)
    x = WL.x_bf16(T, K, WL.W_OLMOE, 90)
    gy = WL.grad_y_bf16(T, N, WL.W_OLMOE, 91)
    off = torch.from_numpy(offsets).to(DEV)
    keys = ("NF4_BM", "NF4_BN", "NF4_CONSUMERS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({"NF4_BM": str(bm), "NF4_BN": str(bn), "NF4_CONSUMERS": str(consumers)})
    try:
        api.nf4_reset_path_counts()
        y = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
        gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
        y2 = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
        gx2 = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
        torch.cuda.synchronize()
        c = api.nf4_path_counts()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert c["grouped_fwd"] == 2 and c["grouped_bwd"] == 2
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "forward not bitwise repeatable"
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)), "input gradient not bitwise repeatable"
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), "grouped y",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, aw), K)
    assert_close(gx, O.grouped_matmul_bwd_input(gyb, offsets, wb), "grouped grad_x",
                 O.grouped_matmul_bwd_input(abs_bits(gyb), offsets, aw), N)


@pytest.mark.parametrize("bm,bn,consumers", [(0, 0, 0), (64, 128, 1), (256, 256, 4), (256, 128, 0),
                                             (128, 128, 5), (128, 128, 6), (128, 256, 6)])
def test_grouped_many_experts(bm, bn, consumers):
    """150 experts (three rounds of the 64-lane expert search), many of them
    empty, several spanning two or three row tiles: every row lands in its
    expert's slice, forward and input gradient, for the default plan and each
    kernel family."""
    E, N, K = 150, 64, 128
    g = np.random.default_rng(150)
    counts = g.integers(0, 12, size=E)
    counts[g.choice(E, 40, replace=False)] = 0
    counts[[3, 70, 140]] = [140, 300, 129]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(offsets[-1])
    wq, wb = _stack(E, N, K, True, 15)
    x = WL.x_bf16(T, K, WL.W_OLMOE, 150)
    gy = WL.grad_y_bf16(T, N, WL.W_OLMOE, 151)
    off = torch.from_numpy(offsets).to(DEV)
    keys = ("NF4_BM", "NF4_BN", "NF4_CONSUMERS")
    saved = {k: os.environ.get(k) for k in keys}
    if consumers or bm:
        os.environ.update({"NF4_BM": str(bm), "NF4_BN": str(bn), "NF4_CONSUMERS": str(consumers)})
    try:
        y = api.nf4_grouped_matmul_fwd(x.to(DEV), off, wq, E)
        gx = api.nf4_grouped_matmul_bwd_input(gy.to(DEV), off, wq, E)
        torch.cuda.synchronize()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    assert_close(y, O.grouped_matmul_fwd(xb, offsets, wb), "150 experts y",
                 O.grouped_matmul_fwd(abs_bits(xb), offsets, aw), K)
    assert_close(gx, O.grouped_matmul_bwd_input(gyb, offsets, wb), "150 experts grad_x",
                 O.grouped_matmul_bwd_input(abs_bits(gyb), offsets, aw), N)
