"""Helpers for the GPU parity tests: move oracle-made quantised weights to the
device, and the tolerance checks of the matmul outputs.

Expected values always come from the oracle on the host; the only thing that
goes to the device from here is input data (oracle-quantised weights, seeded
activations)."""

from __future__ import annotations

import numpy as np
import torch

import workloads as WL
from nf4_bit_weight_amd.api import NF4Weight
from oracle import nf4_oracle as O

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# Matmul acceptance against the oracle's bf16 output (the exact product rounded
# once to bf16): relative Frobenius error and a per-element bound.
REL_FRO = 2e-3
ELEM = 1e-2
# Rigorous per-element bound against the unrounded fp64 product p:
#   |g - p| <= 2^-8 (|p| + e) + e,  e = K * 2^-22 * sum_k |x_k w_k|
# (bf16 RNE relative error 2^-8; fp32 accumulation error of a K-term sum taken
# with four times the textbook K * 2^-24 allowance for any summation order).
U_BF16 = 2.0 ** -8


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def code_tensors(nested: bool):
    """The code tables are call inputs; both sides take them from workloads."""
    code = to_dev(WL.nf4_code_np())
    ncode = to_dev(WL.nested_code_np()) if nested else None
    return code, ncode


def upload(ref: dict, N: int, K: int, nested: bool) -> NF4Weight:
    """NF4Weight on the device holding the oracle's own quantisation."""
    code, ncode = code_tensors(nested)
    if nested:
        return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]),
                         to_dev(ref["nested_absmax"]),
                         to_dev(np.array([ref["nested_offset"]], np.float32)), code, ncode, N, K)
    return NF4Weight(to_dev(ref["packed"]), to_dev(ref["absmax"]), None, None, code, None, N, K)


def ref_bits(ref: dict, shape) -> np.ndarray:
    """Oracle's dequantised bf16 weight bits in the given shape."""
    return O.dequantize_nf4_bf16_bits(ref["packed"], ref["absmax"], ref["nested_absmax"],
                                      ref["nested_offset"]).reshape(shape)


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def abs_bits(b: np.ndarray) -> np.ndarray:
    """|v| of bf16 bit patterns (clear the sign bit)."""
    return (np.asarray(b, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def assert_close(got: torch.Tensor, want64: np.ndarray, what: str, absprod=None, K=None):
    """got: bf16 device output; want64: oracle fp64 product; absprod: oracle
    product of |operands| (enables the rigorous per-element bound)."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == want64.shape, (what, g.shape, want64.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    ref = O.bf16_bits_to_f32(O.bf16_rne_bits_from_f64(want64)).astype(np.float64)
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / (nrm if nrm > 0 else 1.0)
    worst = np.max(np.abs(g - ref) - ELEM * (np.abs(ref) + 1.0)) if g.size else -1
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert worst <= 0, f"{what}: per-element bound exceeded by {worst:.3e}"
    if absprod is not None:
        e = K * 2.0 ** -22 * absprod
        bound = U_BF16 * (np.abs(want64) + e) + e
        over = np.abs(g - want64) - bound
        assert np.max(over) <= 0, f"{what}: exceeds the rounding bound by {np.max(over):.3e}"
    return rel
