"""Parity on the benchmark's own Llama-3.1-8B stack: layers 0 and 31, every
projection, with the weights and inputs drawn on the device by the same seeded
generators and seeds the benchmark uses.

The fp32 weight the generator drew is copied to the host and quantised by the
oracle: the device quantisation must match it byte for byte (packed nibbles,
nested scales, offset).  The fused forward and input gradient of the
benchmark's launch configuration (M = 512, nested, the planner's tiles and
splits) are compared with the oracle's product on 48 sampled rows, every
column, and repeated bitwise.
"""

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, code_tensors, ref_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layer", [0, WL.LLAMA_LAYERS - 1])
@pytest.mark.parametrize("idx", range(len(WL.LLAMA_8B)))
def test_bench_stack_layer(layer, idx):
    p = WL.LLAMA_8B[idx]
    M = WL.LLAMA_M
    code, ncode = code_tensors(True)
    w = WL.gpu_weight_f32(p.N, p.K, seed=WL.stack_weight_seed(WL.LLAMA_STACK_W_SEED, layer, idx), device=DEV)
    wq = api.nf4_quantize(w, code, ncode)
    ref = O.quantize_nf4(w.cpu().numpy(), nested=True)
    del w
    assert np.array_equal(wq.packed.cpu().numpy(), ref["packed"]), "packed nibbles"
    assert np.array_equal(wq.absmax.cpu().numpy(), ref["absmax"]), "nested scale codes"
    assert np.array_equal(wq.nested_absmax.cpu().numpy(), ref["nested_absmax"]), "nested absmax"
    assert wq.nested_offset.cpu().numpy()[0] == ref["nested_offset"], "nested offset"
    wb = ref_bits(ref, (p.N, p.K))
    del ref
    x = WL.gpu_normal_bf16(M, p.K, seed=WL.stack_x_seed(WL.LLAMA_STACK_IN_SEED, layer, WL.X_SLOT[idx]),
                           device=DEV)
    gy = WL.gpu_normal_bf16(M, p.N, seed=WL.stack_gy_seed(WL.LLAMA_STACK_IN_SEED, layer, idx), device=DEV)
    ws = torch.empty(max(16, api.nf4_workspace_bytes(1, M, p.N, p.K), api.nf4_workspace_bytes(2, M, p.N, p.K)),
                     dtype=torch.uint8, device=DEV)
    y = api.nf4_matmul_fwd(x, wq, ws=ws)
    gx = api.nf4_matmul_bwd_input(gy, wq, ws=ws)
    rows = np.sort(np.random.default_rng(100 * layer + idx).choice(M, size=48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    xb = x.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    gyb = gy.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    aw = abs_bits(wb)
    r = torch.from_numpy(rows).to(DEV)
    assert_close(y[r], O.matmul_fwd(xb, wb), f"layer {layer} {p.name} y", O.matmul_fwd(abs_bits(xb), aw), p.K)
    assert_close(gx[r], O.matmul_bwd_input(gyb, wb), f"layer {layer} {p.name} grad_x",
                 O.matmul_bwd_input(abs_bits(gyb), aw), p.N)
    y2 = api.nf4_matmul_fwd(x, wq, ws=ws)
    gx2 = api.nf4_matmul_bwd_input(gy, wq, ws=ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))
