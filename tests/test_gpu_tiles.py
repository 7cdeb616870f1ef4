"""Every tile variant of the fused kernels, forced through the planner's
documented tuning overrides (NF4_BM, NF4_BN, NF4_CONSUMERS, NF4_SPLITS), against the oracle:
bit-exact identity probes and tolerance on ragged shapes, split and unsplit."""

import os

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, bits_of, ref_bits, upload

pytestmark = pytest.mark.gpu

# (rows, columns, kernel choice).  256 x 256: 0 = default (register-operand
# forward, ping-pong input gradient), 4 = ping-pong for both, 2 = producer /
# consumer kernel; 256 x 128 is the 4-wave register-operand forward (the input
# gradient falls back to 256 x 256).  Smaller tiles: MFMA waves per SIMD beside
# the expanding wave; 5 = the register-staged tile kernel (128 columns, 128,
# 64 or 32 rows), 6 = the same with 8 waves (128 or 64 rows, or 128 x 256).
TILES = [(256, 256, 0), (256, 128, 0), (256, 256, 4), (256, 256, 2), (128, 256, 1), (128, 256, 2),
         (64, 256, 1), (128, 128, 1), (64, 128, 1), (128, 128, 5), (64, 128, 5), (32, 128, 5),
         (128, 128, 6), (64, 128, 6), (128, 256, 6)]


@pytest.fixture
def plan_override():
    saved = {k: os.environ.get(k) for k in ("NF4_BM", "NF4_BN", "NF4_SPLITS", "NF4_CONSUMERS")}

    def set_(bm, bn, consumers, splits=0):
        os.environ["NF4_BM"], os.environ["NF4_BN"] = str(bm), str(bn)
        os.environ["NF4_SPLITS"], os.environ["NF4_CONSUMERS"] = str(splits), str(consumers)

    yield set_
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


@pytest.mark.parametrize("bm,bn,consumers", TILES)
def test_tile_identity(bm, bn, consumers, plan_override):
    plan_override(bm, bn, consumers)
    N, K = 320, 384
    w = WL.weight_f32(N, K, WL.W_TINY, 500 + bm + bn)
    ref = O.quantize_nf4(w, nested=True)
    wq = upload(ref, N, K, True)
    wb = ref_bits(ref, (N, K))
    y = api.nf4_matmul_fwd(torch.eye(K, dtype=torch.bfloat16, device=DEV), wq)
    assert np.array_equal(bits_of(y), wb.T)
    gx = api.nf4_matmul_bwd_input(torch.eye(N, dtype=torch.bfloat16, device=DEV), wq)
    assert np.array_equal(bits_of(gx), wb)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("bm,bn,consumers", TILES)
@pytest.mark.parametrize("M,N,K", [(200, 392, 704), (513, 136, 1088)])
def test_tile_vs_oracle(M, N, K, bm, bn, consumers, splits, plan_override):
    plan_override(bm, bn, consumers, splits)
    w = WL.weight_f32(N, K, WL.W_TINY, 600 + M)
    ref = O.quantize_nf4(w, nested=(M % 2 == 0))
    wq = upload(ref, N, K, M % 2 == 0)
    wb = ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, 601)
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, 602)
    xb, gyb, aw = WL.bf16_bits(x), WL.bf16_bits(gy), abs_bits(wb)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert_close(y, O.matmul_fwd(xb, wb), "y", O.matmul_fwd(abs_bits(xb), aw), K)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert_close(gx, O.matmul_bwd_input(gyb, wb), "grad_x", O.matmul_bwd_input(abs_bits(gyb), aw), N)


@pytest.mark.parametrize("bn", [256, 128])
@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("K", [64, 128, 192, 256, 320, 448])
def test_register_operand_forward_step_counts(K, nested, bn, plan_override):
    """The register-operand forward runs its steps three at a time: 1, 2, 3,
    4, 5 and 7 steps per workgroup, ragged rows and columns, against the oracle."""
    plan_override(256, bn, 0, 1)
    M, N = 300, 264
    w = WL.weight_f32(N, K, WL.W_TINY, 700 + K)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    wb = ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, 701 + K)
    xb = WL.bf16_bits(x)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert_close(y, O.matmul_fwd(xb, wb), f"y K={K}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("bn", [128, 256])
def test_register_operand_forward_repeats_bitwise(bn, plan_override):
    """Regression: each copy wait of the register-operand forward must cover
    the whole activation copy of its step for both wave counts (a short wait
    let a step read a half-landed stage).  Many steps per workgroup, several
    launches, every output bitwise equal, sampled columns against the oracle."""
    plan_override(256, bn, 0, 1)
    M, N, K = 256, 1024, 4096
    w = WL.weight_f32(N, K, WL.W_TINY, 900 + bn)
    ref = O.quantize_nf4(w, nested=True)
    wq = upload(ref, N, K, True)
    x = WL.x_bf16(M, K, WL.W_TINY, 901)
    xd = x.to(DEV)
    y0 = api.nf4_matmul_fwd(xd, wq).clone()
    for _ in range(8):
        y = api.nf4_matmul_fwd(xd, wq)
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), "not bitwise repeatable"
    cols = np.sort(np.random.default_rng(bn).choice(N, size=48, replace=False))
    wb = ref_bits(ref, (N, K))[cols]
    xb = WL.bf16_bits(x)
    assert_close(y0[:, torch.from_numpy(cols).to(DEV)], O.matmul_fwd(xb, wb), "sampled",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)


# Tiles served by the producer / consumer kernel.  Its copy rings (2 or 4
# activation stages, 2 or 4 packed-weight slots, by tile and direction) repeat
# with a period of 4 steps, and its step loop is unrolled by 4.
RING_TILES = [(256, 256, 2), (128, 256, 1), (128, 256, 2), (64, 256, 1), (128, 128, 1), (64, 128, 1)]
# The ping-pong kernel (256 x 256, consumers 4; with 0 the input gradient
# only): its weight copies run three steps ahead through three slots, and the
# last steps issue no copies, so its short contractions need the same sweep.
PP_TILES = [(256, 256, 4), (256, 256, 0)]
# The register-staged tile kernel (4 or 8 waves): 128-deep steps, the next step's operands
# held in registers, two LDS buffers.
STAGED_TILES = [(128, 128, 5), (64, 128, 5), (32, 128, 5), (128, 128, 6), (64, 128, 6), (128, 256, 6)]


@pytest.mark.parametrize("steps", [1, 2, 3, 4, 5, 6, 7, 10, 11, 13])
@pytest.mark.parametrize("bm,bn,consumers", RING_TILES + PP_TILES + STAGED_TILES)
def test_tiled_step_counts(steps, bm, bn, consumers, plan_override):
    """One workgroup's contraction of 1 to 13 steps in both directions: every
    remainder of the unrolled step loop with and without a whole period, and
    fewer steps than the copy rings hold; the last step is ragged where the
    step is deeper than one 64-block."""
    plan_override(bm, bn, consumers, 1)
    bk = 16384 // bn                                  # contraction depth of one step
    M, nested = 96, steps % 2 == 1
    seed = 700 + 16 * steps + bm // 64 + bn // 128 + consumers
    # forward: the contraction runs over K
    N, K = 136, steps * bk - (64 if bk == 128 else 0)
    w = WL.weight_f32(N, K, WL.W_TINY, seed)
    ref = O.quantize_nf4(w, nested=nested)
    wq, wb = upload(ref, N, K, nested), ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_TINY, seed + 1)
    xb = WL.bf16_bits(x)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    torch.cuda.synchronize()
    c = api.nf4_path_counts()
    assert c["fwd_tiled"] == 1 and c["splitk_reduce"] == 0
    assert_close(y, O.matmul_fwd(xb, wb), f"y steps={steps}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    # input gradient: the contraction runs over N
    N, K = steps * bk - 8, 192
    w = WL.weight_f32(N, K, WL.W_TINY, seed + 2)
    ref = O.quantize_nf4(w, nested=nested)
    wq, wb = upload(ref, N, K, nested), ref_bits(ref, (N, K))
    gy = WL.grad_y_bf16(M, N, WL.W_TINY, seed + 3)
    gyb = WL.bf16_bits(gy)
    gx = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    gx2 = api.nf4_matmul_bwd_input(gy.to(DEV), wq)
    assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16)), "not bitwise repeatable"
    assert_close(gx, O.matmul_bwd_input(gyb, wb), f"grad_x steps={steps}",
                 O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb)), N)


def _weights(N, K, seed):
    w = WL.weight_f32(N, K, WL.W_TINY, seed)
    ref = O.quantize_nf4(w, nested=True)
    return upload(ref, N, K, True), ref_bits(ref, (N, K))


@pytest.mark.parametrize("bm,bn,consumers", [(256, 256, 0), (256, 128, 0), (256, 256, 4), (128, 128, 1),
                                             (64, 128, 1), (128, 128, 6), (128, 256, 6)])
@pytest.mark.parametrize("steps", [1, 2, 3])
def test_nested_first_steps_repeat(bm, bn, consumers, steps, plan_override):
    """Nested statistics and contractions of one to three steps, so every read
    of a copied scale comes right after the prologue: a hundred launches in a
    row are bitwise equal in both directions and the first matches the
    oracle.  (Consecutive steps' nested scales share an address; no counted
    wait may pass before the older copy of it has landed.)"""
    plan_override(bm, bn, consumers, 1)
    bk = 64 if 256 in (bm, bn) else 128                # contraction depth of one step
    M, N, K = 200, 392, steps * bk
    wq, wb = _weights(N, K, 1200 + 10 * steps + consumers)
    x = WL.x_bf16(M, K, WL.W_TINY, 1201 + steps)
    xd = x.to(DEV)
    ys = [api.nf4_matmul_fwd(xd, wq) for _ in range(100)]
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), f"forward call {i} differs"
    xb = WL.bf16_bits(x)
    assert_close(ys[0], O.matmul_fwd(xb, wb), "y", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
    N2, K2 = steps * bk, 192
    wq2, wb2 = _weights(N2, K2, 1300 + 10 * steps + consumers)
    gy = WL.grad_y_bf16(M, N2, WL.W_TINY, 1301 + steps)
    gyd = gy.to(DEV)
    gs = [api.nf4_matmul_bwd_input(gyd, wq2) for _ in range(100)]
    torch.cuda.synchronize()
    for i, g in enumerate(gs):
        assert torch.equal(g.view(torch.int16), gs[0].view(torch.int16)), f"input gradient call {i} differs"
    gyb = WL.bf16_bits(gy)
    assert_close(gs[0], O.matmul_bwd_input(gyb, wb2), "grad_x", O.matmul_bwd_input(abs_bits(gyb), abs_bits(wb2)), N2)
