"""GPU parity of the fused NF4 forward and input gradient against the oracle.

* identity / permutation probes: the in-register expansion equals the
  oracle's bf16 W_hat bit for bit, in both orientations;
* seeded tolerance checks across tile boundaries, ragged tails, every tile
  height, split and unsplit contractions, plain and nested statistics;
* full-size Llama-3.1-8B (M = 512) and Qwen-32B (M = 2048) projections in the
  same launch configuration the benchmark times, checked on sampled rows;
* bitwise run-to-run determinism.
"""

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, bits_of, ref_bits, upload

pytestmark = pytest.mark.gpu


def _setup(M, N, K, nested, seed):
    w = WL.weight_f32(N, K, WL.W_TINY, 1000 + seed)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    wb = ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, 1000 + seed)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 1000 + seed)
    return wq, wb, x, gy


def test_tiny_linear_fwd_bwd():
    """The tiny NF4 linear: x [64, 256], W [128, 256] non-nested."""
    M, N, K = WL.TINY_M, WL.TINY_N, WL.TINY_K
    w = WL.weight_f32(N, K, WL.W_TINY, 0)
    ref = O.quantize_nf4(w)
    wq = upload(ref, N, K, False)
    wb = ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, 0)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 0)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    xb, gyb = WL.bf16_bits(x), WL.bf16_bits(gy)
    assert_close(y, O.matmul_fwd(xb, wb), "y", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    assert_close(gx, O.matmul_bwd_input(gyb, wb), "grad_x",
                 O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb)), N)
    y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx2 = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("N,K", [(256, 256), (320, 192), (136, 512)])
def test_identity_probe(N, K, nested):
    """x = I_K gives y = W_hat^T and grad_y = I_N gives grad_x = W_hat, bit for
    bit (one non-zero product per output element)."""
    w = WL.weight_f32(N, K, WL.W_TINY, 7 * N + K)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    wb = ref_bits(ref, (N, K))
    eye_k = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    eye_n = torch.eye(N, dtype=torch.bfloat16, device=DEV)
    y = api.nf4_matmul_fwd(eye_k, wq)
    assert np.array_equal(bits_of(y), wb.T), "forward identity probe"
    gx = api.nf4_matmul_bwd_input(eye_n, wq)
    assert np.array_equal(bits_of(gx), wb), "input-gradient identity probe"


@pytest.mark.parametrize("M", [1, 64, 100, 256, 700])
def test_permutation_probe(M):
    """Rows of x are unit vectors e_p(m): y[m] = W_hat[:, p(m)] exactly, at
    every tile height the planner picks."""
    N, K = 264, 320
    w = WL.weight_f32(N, K, WL.W_TINY, 31 + M)
    ref = O.quantize_nf4(w, nested=True)
    wq = upload(ref, N, K, True)
    wb = ref_bits(ref, (N, K))
    p = np.random.default_rng(M).integers(0, K, size=M)
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[np.arange(M), p] = 1.0
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert np.array_equal(bits_of(y), wb.T[p])
    q = np.random.default_rng(M + 1).integers(0, N, size=M)
    gy = torch.zeros((M, N), dtype=torch.bfloat16)
    gy[np.arange(M), q] = 1.0
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert np.array_equal(bits_of(gx), wb[q])


def test_scaled_identity_weight():
    """W = 2 * I (one non-zero per block row): y = 2 x exactly."""
    N = K = 128
    w = (np.eye(N, dtype=np.float32) * 2).astype(np.float32)
    ref = O.quantize_nf4(w)
    wq = upload(ref, N, K, False)
    x = WL.x_bf16(96, K, WL.W_TINY, 5)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert torch.equal(y.cpu().view(torch.int16), (x * 2).view(torch.int16))


SHAPES = [
    (1, 64, 64), (33, 200, 128), (65, 136, 320), (130, 264, 192), (300, 512, 512),
    (513, 1024, 256), (64, 256, 4096), (200, 128, 2048), (256, 2048, 1024),
]


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matmul_vs_oracle(M, N, K, nested):
    wq, wb, x, gy = _setup(M, N, K, nested, M + N + K)
    xb, gyb = WL.bf16_bits(x), WL.bf16_bits(gy)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert_close(y, O.matmul_fwd(xb, wb), f"y {M}x{N}x{K}",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert_close(gx, O.matmul_bwd_input(gyb, wb), f"grad_x {M}x{N}x{K}",
                 O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb)), N)


def test_split_contraction_is_used_and_exact_enough():
    M, N, K = 64, 256, 4096          # one output tile -> the contraction is split
    assert api.nf4_workspace_bytes(1, M, N, K) > 0
    wq, wb, x, gy = _setup(M, N, K, True, 77)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    torch.cuda.synchronize()
    c = api.nf4_path_counts()
    assert c["splitk_reduce"] == 1 and c["fwd_tiled"] == 1
    assert_close(y, O.matmul_fwd(WL.bf16_bits(x), wb), "split y")


def test_determinism_repeat_and_streams():
    M, N, K = 384, 1024, 2048
    wq, wb, x, gy = _setup(M, N, K, True, 99)
    xd, gyd = x.to(DEV), gy.to(DEV)
    y0 = api.nf4_matmul_fwd(xd, wq).clone()
    g0 = api.nf4_matmul_bwd_input(gyd, wq).clone()
    junk = torch.randn(4096, 4096, device=DEV) @ torch.randn(4096, 4096, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = api.nf4_matmul_fwd(xd, wq)
        g1 = api.nf4_matmul_bwd_input(gyd, wq)
    torch.cuda.synchronize()
    del junk
    for _ in range(3):
        assert torch.equal(api.nf4_matmul_fwd(xd, wq).view(torch.int16), y0.view(torch.int16))
        assert torch.equal(api.nf4_matmul_bwd_input(gyd, wq).view(torch.int16), g0.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    assert torch.equal(g1.view(torch.int16), g0.view(torch.int16))


def _full_size(projs, idx, M, wl, sample_rows=48):
    p = projs[idx]
    w = WL.weight_f32(p.N, p.K, wl, 0, idx)
    ref = O.quantize_nf4(w, nested=True)
    del w
    wq = upload(ref, p.N, p.K, True)
    wb = ref_bits(ref, (p.N, p.K))
    x = WL.x_bf16(M, p.K, wl, 0)
    gy = WL.grad_y_bf16(M, p.N, wl, 0, idx)
    rows = np.sort(np.random.default_rng(idx).choice(M, size=sample_rows, replace=False))
    rows[0], rows[-1] = 0, M - 1
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    xb, gyb = WL.bf16_bits(x), WL.bf16_bits(gy)
    aw = abs_bits(wb)
    assert_close(y[rows], O.matmul_fwd(xb[rows], wb), f"{p.name} y",
                 O.matmul_fwd(abs_bits(xb[rows]), aw), p.K)
    assert_close(gx[rows], O.matmul_bwd_input(gyb[rows], wb), f"{p.name} grad_x",
                 O.matmul_bwd_input(abs_bits(gyb[rows]), aw), p.N)
    y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx2 = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "fwd not bitwise repeatable"
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)), "bwd not bitwise repeatable"


@pytest.mark.parametrize("idx", range(7))
def test_llama_projection_m512(idx):
    _full_size(WL.LLAMA_8B, idx, WL.LLAMA_M, WL.W_LLAMA)


@pytest.mark.parametrize("idx", [0, 1, 4, 6])          # q/o, k/v, gate/up, down: each distinct shape
def test_qwen_projection_m2048(idx):
    _full_size(WL.QWEN_32B, idx, WL.QWEN_M, WL.W_QWEN, sample_rows=64)   # 8 per 256-row tile
