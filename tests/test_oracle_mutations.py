"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle module (the kind a reimplementation
from the pages could make: a tie rule, the nibble order, a dropped halving, a
block index, a nested-decode step, a transposed operand, a rounding mode, an
expert slice, a summation order) and runs every pin of test_oracle_pins
against the mutated oracle.  At least one pin must fail for each mutant; the
unmutated oracle passes them all.  The mutants are planted here, on the CPU,
and undone after each case.
"""

import inspect

import numpy as np
import pytest

from oracle import nf4_oracle as O
import test_oracle_pins as P

F32, F64 = np.float32, np.float64


def _pins():
    """(name, zero-argument callable) for every pin, parametrised ones expanded."""
    out = []
    for name, fn in sorted(vars(P).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        argnames, values = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            out.append((f"{name}{v}", (lambda fn=fn, kw=dict(zip(names, v)): fn(**kw))))
    return out


PINS = _pins()


def _failing_pins():
    failed = []
    for name, fn in PINS:
        try:
            fn()
        except Exception:                      # a failed assertion or a crash both count
            failed.append(name)
    return failed


# ---- the mutants (each returns the replacement functions) -------------------

def _tie_rule():
    def nearest_index(t, mids):
        t = np.asarray(t, dtype=F32)
        out = np.zeros(t.shape, dtype=np.int64)
        for m in mids:
            out += (t >= m)                     # ties go up instead of down
        return out
    return {"nearest_index": nearest_index}


def _nibble_order():
    # low nibble first, consistently in both directions (round trips still pass)
    def pack_nibbles(q):
        q = np.asarray(q, dtype=np.uint8)
        return ((q[1::2] << 4) | q[0::2]).astype(np.uint8)

    def unpack_nibbles(packed):
        p = np.asarray(packed, dtype=np.uint8)
        q = np.empty(p.shape[0] * 2, dtype=np.uint8)
        q[0::2] = p & 0x0F
        q[1::2] = p >> 4
        return q
    return {"pack_nibbles": pack_nibbles, "unpack_nibbles": unpack_nibbles}


def _midpoint_not_halved():
    def midpoints(code):
        c = np.asarray(code, dtype=F32)
        return (c[:-1] + c[1:]).astype(F32)
    return {"midpoints": midpoints}


def _neighbour_block_scale():
    orig = O.dequantize_nf4_f32

    def dequantize_nf4_f32(packed, absmax, nested_absmax=None, nested_offset=None,
                           code=None, nested_code=None, n_elems=None):
        code = O.nf4_code() if code is None else np.asarray(code, dtype=F32)
        q = O.unpack_nibbles(packed).astype(np.int64)
        if n_elems is not None:
            q = q[:n_elems]
        scale = O.decode_absmax(absmax, nested_absmax, nested_offset, nested_code)
        blk = np.minimum(np.arange(q.shape[0]) // O.BLOCK + 1, scale.shape[0] - 1)
        return (code[q] * scale[blk]).astype(F32)
    assert orig is not None
    return {"dequantize_nf4_f32": dequantize_nf4_f32}


def _nested_offset_dropped():
    def decode_absmax(absmax, nested_absmax=None, nested_offset=None, nested_code=None):
        if nested_absmax is None:
            return np.asarray(absmax, dtype=F32)
        ncode = O.uniform_nested_code() if nested_code is None else np.asarray(nested_code, dtype=F32)
        q2 = np.asarray(absmax, dtype=np.uint8).astype(np.int64)
        s2 = np.asarray(nested_absmax, dtype=F32)
        g = np.arange(q2.shape[0]) // O.NESTED_BLOCK
        return (ncode[q2] * s2[g]).astype(F32)
    return {"decode_absmax": decode_absmax}


def _nested_group_index():
    def decode_absmax(absmax, nested_absmax=None, nested_offset=None, nested_code=None):
        if nested_absmax is None:
            return np.asarray(absmax, dtype=F32)
        ncode = O.uniform_nested_code() if nested_code is None else np.asarray(nested_code, dtype=F32)
        q2 = np.asarray(absmax, dtype=np.uint8).astype(np.int64)
        s2 = np.asarray(nested_absmax, dtype=F32)
        g = np.arange(q2.shape[0]) // O.BLOCK           # 64 instead of 256 per group
        g = np.minimum(g, s2.shape[0] - 1)
        prod = (ncode[q2] * s2[g]).astype(F32)
        return (prod + F32(nested_offset)).astype(F32)
    return {"decode_absmax": decode_absmax}


def _offset_in_float32():
    def absmax_mean_offset(absmax):
        a = np.asarray(absmax, dtype=F32)
        acc = F32(0)
        for v in a:                                     # running fp32 sum
            acc = F32(acc + v)
        return F32(acc / F32(a.shape[0]))
    return {"absmax_mean_offset": absmax_mean_offset}


def _signed_block_max():
    def _blockwise_absmax(flat, block):
        n = flat.shape[0]
        nb = -(-n // block)
        pad = nb * block - n
        a = np.asarray(flat)
        if pad:
            a = np.concatenate([a, np.zeros(pad, dtype=a.dtype)])
        return a.reshape(nb, block).max(axis=1)         # max w, not max |w|
    return {"_blockwise_absmax": _blockwise_absmax}


def _fwd_without_transpose():
    def matmul_fwd(x_bf16_bits, w_bf16_bits):
        x = O._as_f64(x_bf16_bits)
        w = O._as_f64(w_bf16_bits)
        return x @ w                                     # W, not W^T
    return {"matmul_fwd": matmul_fwd}


def _bwd_with_transpose():
    def matmul_bwd_input(gy_bf16_bits, w_bf16_bits):
        gy = O._as_f64(gy_bf16_bits)
        w = O._as_f64(w_bf16_bits)
        return gy @ w.T                                  # W^T instead of W
    return {"matmul_bwd_input": matmul_bwd_input}


def _bf16_truncation():
    def bf16_rne_bits(x):
        u = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
        return (u >> 16).astype(np.uint16)               # truncate, no rounding
    return {"bf16_rne_bits": bf16_rne_bits}


def _output_rounded_twice():
    def bf16_rne_bits_from_f64(x):
        f = np.ascontiguousarray(x, dtype=F64).astype(F32)   # through fp32 first
        u = f.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return {"bf16_rne_bits_from_f64": bf16_rne_bits_from_f64}


def _wrong_expert():
    def grouped_matmul_fwd(x_bf16_bits, offsets, w_stack_bf16_bits):
        E, N, K = w_stack_bf16_bits.shape
        out = np.zeros((x_bf16_bits.shape[0], N), dtype=F64)
        for e in range(E):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi > lo:
                out[lo:hi] = O.matmul_fwd(x_bf16_bits[lo:hi], w_stack_bf16_bits[(e + 1) % E])
        return out
    return {"grouped_matmul_fwd": grouped_matmul_fwd}


def _code_sign_flipped():
    base = O.nf4_code

    def nf4_code():
        return (-base()[::-1]).astype(F32)                # mirrored table
    return {"nf4_code": nf4_code}


MUTANTS = {
    "tie_rule": _tie_rule,
    "nibble_order": _nibble_order,
    "midpoint_not_halved": _midpoint_not_halved,
    "neighbour_block_scale": _neighbour_block_scale,
    "nested_offset_dropped": _nested_offset_dropped,
    "nested_group_index": _nested_group_index,
    "offset_in_float32": _offset_in_float32,
    "signed_block_max": _signed_block_max,
    "fwd_without_transpose": _fwd_without_transpose,
    "bwd_with_transpose": _bwd_with_transpose,
    "bf16_truncation": _bf16_truncation,
    "output_rounded_twice": _output_rounded_twice,
    "wrong_expert": _wrong_expert,
    "code_sign_flipped": _code_sign_flipped,
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]().items():
        assert hasattr(O, attr) and inspect.isfunction(getattr(O, attr)), attr
        monkeypatch.setattr(O, attr, fn)
    failed = _failing_pins()
    assert failed, f"no pin catches the planted mistake {name!r}"
