"""GPU edge cases of the fused calls, against the oracle.

* empty batches (M = 0, total_M = 0) through the binding: empty outputs, no
  launch (the path counters stay at zero), including torch's NULL pointers of
  empty tensors;
* all-zero weights, plain and nested (block scales 0; nested, every block
  decodes to the offset 0): the outputs are exactly +-0 on every path (the
  small-M streaming kernel, the tiled kernels, split contractions, grouped);
* the narrowest shapes the format allows: K = 64 (one block per row) and
  N = 8, at decode and large M.
"""

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, ref_bits, upload

pytestmark = pytest.mark.gpu


def _weight(N, K, nested, seed, zero=False):
    w = np.zeros((N, K), np.float32) if zero else WL.weight_f32(N, K, WL.W_TINY, 500 + seed)
    ref = O.quantize_nf4(w, nested=nested)
    return upload(ref, N, K, nested), ref_bits(ref, (N, K))


@pytest.mark.parametrize("nested", [False, True])
def test_empty_batches(nested):
    N, K = 256, 512
    wq, _ = _weight(N, K, nested, 1)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(torch.empty((0, K), dtype=torch.bfloat16, device=DEV), wq)
    gx = api.nf4_matmul_bwd_input(torch.empty((0, N), dtype=torch.bfloat16, device=DEV), wq)
    E = 4
    wg, _ = _weight(E * 64, K, nested, 2)
    wge = wg.per_expert(E)
    off = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    yg = api.nf4_grouped_matmul_fwd(torch.empty((0, K), dtype=torch.bfloat16, device=DEV), off, wge, E)
    gxg = api.nf4_grouped_matmul_bwd_input(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), off, wge, E)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, N) and tuple(gx.shape) == (0, K)
    assert tuple(yg.shape) == (0, 64) and tuple(gxg.shape) == (0, K)
    assert all(v == 0 for v in api.nf4_path_counts().values())


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M", [1, 8, 32, 64, 512])
def test_all_zero_weight(M, nested):
    N, K = 384, 1024
    wq, wb = _weight(N, K, nested, 3, zero=True)
    assert not np.any(O.bf16_bits_to_f32(wb))
    x = WL.x_bf16(M, K, WL.W_TINY, 600 + M).to(DEV)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 600 + M).to(DEV)
    y = api.nf4_matmul_fwd(x, wq)
    gx = api.nf4_matmul_bwd_input(gy, wq)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0
    assert torch.count_nonzero(gx.float()) == 0


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (3, 1000, 64), (512, 8, 64), (700, 24, 64),
                                   (512, 2048, 64), (1, 8, 4096), (600, 8, 2048)])
def test_narrow_shapes(M, N, K, nested):
    wq, wb = _weight(N, K, nested, M + N + K)
    x = WL.x_bf16(M, K, WL.W_TINY, 700 + M)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 700 + M)
    xb, gyb = WL.bf16_bits(x), WL.bf16_bits(gy)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert_close(y, O.matmul_fwd(xb, wb), f"y {M}x{N}x{K}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    assert_close(gx, O.matmul_bwd_input(gyb, wb), f"gx {M}x{N}x{K}",
                 O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb)), N)


@pytest.mark.parametrize("nested", [False, True])
def test_empty_contraction_zero_fill(nested):
    """N = 0 (forward) or K = 0 (input gradient) with rows present: the output
    is all zeros, written by a fill kernel (replayed from a HIP graph too)."""
    M, K = 37, 128
    wq, _ = _weight(64, K, nested, 9)
    w0 = api.NF4Weight(wq.packed[:0], wq.absmax[:0],
                       wq.nested_absmax[:0] if nested else None, wq.nested_offset,
                       wq.code, wq.nested_code, 0, K)
    x = torch.randn((M, K), device=DEV).to(torch.bfloat16)
    y = torch.full((M, 0), 1.0, dtype=torch.bfloat16, device=DEV)
    assert tuple(api.nf4_matmul_fwd(x, w0, out=y).shape) == (M, 0)
    gx = torch.full((M, K), 7.0, dtype=torch.bfloat16, device=DEV)
    g = torch.empty((M, 0), dtype=torch.bfloat16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.nf4_matmul_bwd_input(g, w0, out=gx)
    for _ in range(3):
        gx.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.count_nonzero(gx.float()) == 0
    gx.fill_(7.0)
    api.nf4_matmul_bwd_input(g, w0, out=gx)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gx.float()) == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_autograd_keeps_caller_dtype(dtype):
    """The wrapper computes in bf16 and hands back the caller's dtype, for the
    output and for the input gradient (plain and grouped)."""
    from nf4_bit_weight_amd.autograd import nf4_grouped_linear, nf4_linear
    N, K, M = 128, 256, 16
    wq, _ = _weight(N, K, True, 11)
    x = torch.randn((M, K), device=DEV, dtype=dtype, requires_grad=True)
    y = nf4_linear(x, wq)
    assert y.dtype == dtype
    y.float().sum().backward()
    assert x.grad.dtype == dtype
    ref = nf4_linear(x.detach().to(torch.bfloat16), wq)
    # the wrapper's output is the bf16 result cast to the caller's dtype: compare
    # after the same cast (bf16 -> fp16 -> bf16 is not exact below 2^-17)
    assert torch.equal(y, ref.to(dtype))
    E = 2
    wg, _ = _weight(E * N, K, True, 12)
    off = torch.tensor([0, 5, M], dtype=torch.int32, device=DEV)
    xg = torch.randn((M, K), device=DEV, dtype=dtype, requires_grad=True)
    yg = nf4_grouped_linear(xg, off, wg.per_expert(E), E)
    assert yg.dtype == dtype
    yg.float().sum().backward()
    assert xg.grad.dtype == dtype
