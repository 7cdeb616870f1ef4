"""Python binding of libnf4.so with the same names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are passed to
the C entry point, and a non-zero status raises NF4Error.  Every step of the
computation runs in the library's HIP kernels; nothing here computes.

Tensor conventions (all on the same CUDA/HIP device, contiguous):
  packed         uint8  [N*K/2]  (any shape with that many bytes); [N*K] for
                 the 8-bit blockwise formats
  absmax         float32 [nb] (plain) or uint8 [nb] (nested)
  nested_absmax  float32 [ng] or None
  nested_offset  float32 [1] or None
  code           float32 [16] (4-bit) or [256] (8-bit)
  nested_code    float32 [256] or None
A weight's `bits` (4 or 8) selects the C entry points: nf4_* or nf4_*_8bit.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: Optional[torch.Tensor], name: str, dtype=None, numel=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


@dataclass
class NF4Weight:
    """One quantised tensor: the W-args of the ABI as separate tensors.

    Every field is a plain tensor so an autograd Function can route it through
    save_for_backward (Soup issue #842, "Design sketch")."""
    packed: torch.Tensor
    absmax: torch.Tensor
    nested_absmax: Optional[torch.Tensor]
    nested_offset: Optional[torch.Tensor]
    code: torch.Tensor
    nested_code: Optional[torch.Tensor]
    N: int
    K: int
    bits: int = 4        # 4: packed nibbles, 16-entry code; 8: one byte, 256-entry code

    @property
    def nested(self) -> bool:
        return self.nested_absmax is not None

    def tensors(self):
        return (self.packed, self.absmax, self.nested_absmax, self.nested_offset,
                self.code, self.nested_code)

    def per_expert(self, E: int) -> "NF4Weight":
        """View of an [E*N, K] stack quantised as one tensor, with N per expert
        (the form the grouped calls take)."""
        if self.N % E:
            raise ValueError(f"{self.N} rows do not split into {E} experts")
        return NF4Weight(*self.tensors(), self.N // E, self.K, self.bits)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors()[:4] if t is not None)


def _check_w(w: NF4Weight, rows: int):
    dev = w.packed.device
    if w.bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, got {w.bits}")
    nb = L.lib().nf4_absmax_count(rows, w.K)
    _need(w.packed, "packed", torch.uint8, rows * w.K // 2 if w.bits == 4 else rows * w.K)
    _need(w.code, "code", torch.float32, 16 if w.bits == 4 else 256, dev)
    if w.nested:
        ng = L.lib().nf4_nested_count(rows, w.K)
        _need(w.absmax, "absmax", torch.uint8, nb, dev)
        _need(w.nested_absmax, "nested_absmax", torch.float32, ng, dev)
        _need(w.nested_offset, "nested_offset", torch.float32, 1, dev)
        _need(w.nested_code, "nested_code", torch.float32, 256, dev)
    else:
        _need(w.absmax, "absmax", torch.float32, nb, dev)


def _wargs(w: NF4Weight):
    return (w.packed.data_ptr(), w.absmax.data_ptr(), _ptr(w.nested_absmax),
            _ptr(w.nested_offset), w.code.data_ptr(),
            _ptr(w.nested_code) if w.nested else None, w.N, w.K)


def nf4_workspace_bytes(op: int, M: int, N: int, K: int, E: int = 1) -> int:
    return int(L.lib().nf4_workspace_bytes(op, M, N, K, E))


def _workspace(op: int, M: int, N: int, K: int, E: int, device, ws: Optional[torch.Tensor]):
    need = nf4_workspace_bytes(op, M, N, K, E)
    if need == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    buf = torch.empty(need, dtype=torch.uint8, device=device)
    return buf, need


def _fn(name: str, bits: int):
    return getattr(L.lib(), name if bits == 4 else name + "_8bit")


def nf4_quantize_8bit(w: torch.Tensor, code: torch.Tensor, nested_code: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> NF4Weight:
    """Quantise w [N, K] to an 8-bit blockwise format: one byte per weight,
    an index into the ascending 256-entry table `code` (int8 map, fp8 e4m3
    codebook, ...), the same 64-element blocks and statistics as NF4."""
    return nf4_quantize(w, code, nested_code, ws, bits=8)


def nf4_quantize(w: torch.Tensor, code: torch.Tensor, nested_code: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None, bits: int = 4) -> NF4Weight:
    """Quantise w [N, K] (fp32 or bf16 device tensor) to NF4 (or, with
    bits=8, to the 8-bit blockwise format of the 256-entry `code`)."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    _need(code, "code", torch.float32, 16 if bits == 4 else 256)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    _need(w, "w")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    N, K = w.shape
    dev = w.device
    lib = L.lib()
    nb = lib.nf4_absmax_count(N, K)
    packed = torch.empty(N * K // 2 if bits == 4 else N * K, dtype=torch.uint8, device=dev)
    nested = nested_code is not None
    if nested:
        absmax = torch.empty(nb, dtype=torch.uint8, device=dev)
        nabs = torch.empty(lib.nf4_nested_count(N, K), dtype=torch.float32, device=dev)
        noff = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
        nabs = noff = None
    wsb, wsn = _workspace(L.NF4_OP_QUANTIZE, 0, N, K, 1, dev, ws) if nested else (None, 0)
    dt = L.NF4_DTYPE_BF16 if w.dtype == torch.bfloat16 else L.NF4_DTYPE_F32
    st = _fn("nf4_quantize", bits)(w.data_ptr(), dt, N, K, code.data_ptr(), _ptr(nested_code),
                                   packed.data_ptr(), absmax.data_ptr(), _ptr(nabs), _ptr(noff),
                                   _ptr(wsb), wsn, _stream())
    L.check("nf4_quantize" if bits == 4 else "nf4_quantize_8bit", st)
    return NF4Weight(packed, absmax, nabs, noff, code, nested_code if nested else None, N, K, bits)


def nf4_dequantize(w: NF4Weight, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Dense W_hat [N, K] in bf16 (or fp32) from the packed weight."""
    _check_w(w, w.N)
    if out is None:
        out = torch.empty((w.N, w.K), dtype=out_dtype, device=w.packed.device)
    _need(out, "out", out_dtype, w.N * w.K)
    dt = L.NF4_DTYPE_BF16 if out_dtype == torch.bfloat16 else L.NF4_DTYPE_F32
    st = _fn("nf4_dequantize", w.bits)(*_wargs(w), dt, out.data_ptr(), _stream())
    L.check("nf4_dequantize", st)
    return out


def nf4_matmul_fwd(x: torch.Tensor, w: NF4Weight, out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x . W_hat^T; x bf16 [M, K] -> y bf16 [M, N]."""
    _check_w(w, w.N)
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [M, {w.K}]")
    _need(x, "x", torch.bfloat16, device=w.packed.device)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, M * w.N)
    op = L.NF4_OP_MATMUL_FWD if w.bits == 4 else L.NF4_OP_MATMUL_FWD_8BIT
    wsb, wsn = _workspace(op, M, w.N, w.K, 1, x.device, ws)
    st = _fn("nf4_matmul_fwd", w.bits)(x.data_ptr(), M, *_wargs(w), out.data_ptr(), _ptr(wsb), wsn,
                                       _stream())
    L.check("nf4_matmul_fwd", st)
    return out


def nf4_matmul_bwd_input(grad_y: torch.Tensor, w: NF4Weight, out: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grad_x = grad_y . W_hat; grad_y bf16 [M, N] -> grad_x bf16 [M, K]."""
    _check_w(w, w.N)
    if grad_y.dim() != 2 or grad_y.shape[1] != w.N:
        raise ValueError(f"grad_y must be [M, {w.N}]")
    _need(grad_y, "grad_y", torch.bfloat16, device=w.packed.device)
    M = grad_y.shape[0]
    if out is None:
        out = torch.empty((M, w.K), dtype=torch.bfloat16, device=grad_y.device)
    _need(out, "out", torch.bfloat16, M * w.K)
    op = L.NF4_OP_MATMUL_BWD_INPUT if w.bits == 4 else L.NF4_OP_MATMUL_BWD_INPUT_8BIT
    wsb, wsn = _workspace(op, M, w.N, w.K, 1, grad_y.device, ws)
    st = _fn("nf4_matmul_bwd_input", w.bits)(grad_y.data_ptr(), M, *_wargs(w), out.data_ptr(),
                                             _ptr(wsb), wsn, _stream())
    L.check("nf4_matmul_bwd_input", st)
    return out


def nf4_grouped_matmul_fwd(x: torch.Tensor, offsets: torch.Tensor, w: NF4Weight, E: int,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-expert y over expert-sorted rows; w is the [E*N, K] stack (N per expert)."""
    _check_w(w, E * w.N)
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [T, {w.K}]")
    _need(x, "x", torch.bfloat16, device=w.packed.device)
    _need(offsets, "offsets", torch.int32, E + 1, x.device)
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, w.N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, T * w.N)
    st = _fn("nf4_grouped_matmul_fwd", w.bits)(x.data_ptr(), offsets.data_ptr(), E, T, *_wargs(w),
                                               out.data_ptr(), None, 0, _stream())
    L.check("nf4_grouped_matmul_fwd", st)
    return out


def nf4_grouped_matmul_bwd_input(grad_y: torch.Tensor, offsets: torch.Tensor, w: NF4Weight,
                                 E: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-expert grad_x over expert-sorted rows."""
    _check_w(w, E * w.N)
    if grad_y.dim() != 2 or grad_y.shape[1] != w.N:
        raise ValueError(f"grad_y must be [T, {w.N}]")
    _need(grad_y, "grad_y", torch.bfloat16, device=w.packed.device)
    _need(offsets, "offsets", torch.int32, E + 1, grad_y.device)
    T = grad_y.shape[0]
    if out is None:
        out = torch.empty((T, w.K), dtype=torch.bfloat16, device=grad_y.device)
    _need(out, "out", torch.bfloat16, T * w.K)
    st = _fn("nf4_grouped_matmul_bwd_input", w.bits)(grad_y.data_ptr(), offsets.data_ptr(), E, T,
                                                     *_wargs(w), out.data_ptr(), None, 0, _stream())
    L.check("nf4_grouped_matmul_bwd_input", st)
    return out


def nf4_path_counts() -> dict:
    lib = L.lib()
    return {name: int(lib.nf4_path_count(i)) for i, name in enumerate(L.PATHS)}


def nf4_reset_path_counts() -> None:
    L.lib().nf4_reset_path_counts()
