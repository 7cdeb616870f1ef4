"""CPU oracle for NF4 blockwise quantisation, dequantisation and the NF4 linear.

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP library; it is
never part of the product path.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it.  It shares no code, table
or helper with the HIP path and imports nothing from it.

Sources (the pages describe the method; they print no NF4 code values, no bit
order and no rounding rule -- the readings taken where they are silent are
listed at each step):

* bitsandbytes issue #2034, "MatMul4Bit keeps B and quant_state on ctx instead
  of save_for_backward ..." -- section "Minimal reproducer" calls
  quantize_4bit(w, blocksize=64, quant_type="nf4", compress_statistics=True)
  and matmul_4bit(h, w.t(), quant_state=st), i.e. y = h . W^T with W in the
  [out, in] layout of F.linear; section "Root cause" gives the backward as
  grad_A = grad_output @ dequantize_4bit(B, state) and names the QuantState
  fields (absmax, offset, code); section "Why save_for_backward fixes it"
  names the double-quantisation fields nested_absmax / nested_offset.
* bitsandbytes fork PR "Experts trainability: bit-exact recompute-in-backward
  + ExpertsNbit", "Commit 1" table: NF4 storage is 4-bit packed, two values per
  byte; "Commit 2": each expert projection is dequantise + F.linear forward
  and grad_output @ W backward on the dequantised expert slice.
* Soup issue #842 "Layer streaming: a checkpoint-visible fused NF4
  dequantise-and-multiply", "Design sketch": the fused backward computes only
  grad_x = grad_y @ W.

Readings where the pages are silent (each is an argument or a documented
constant, identical on both sides of the parity check):

R1  NF4 code: 16 ascending fp32 values, passed in.  `nf4_code()` holds the
    4-decimal NormalFloat-4 levels.
R2  Packing: flattened row-major, element 2i in the HIGH nibble of byte i.
R3  Blocks: 64 consecutive flattened elements; the last may be partial.
R4  Nearest code: thresholds at fp32 midpoints of adjacent codes; the code
    index is the number of midpoints strictly below t, so an exact midpoint
    rounds to the lower code.  t = w / absmax with one correctly rounded fp32
    division; an all-zero block gives t = 0.
R5  Double quantisation: offset = mean of the fp32 absmax array, summed in
    fp64 in a fixed order (sequential within consecutive chunks of 256, then
    the chunk sums sequentially), divided in fp64 and rounded to fp32;
    c = fp32(absmax - offset); groups of 256 c's get an fp32 scale
    s2 = max|c| and an 8-bit index by R4 against a 256-entry table.
R6  Nested table: passed in; `uniform_nested_code()` is the symmetric uniform
    table (2j - 255) / 255.
R7  Decode: absmax_hat = fp32(fp32(nested_code[q2] * s2) + offset) (two
    roundings, no fused multiply-add); w_hat = fp32(code[q] * absmax_hat);
    the compute-dtype weight is bf16 by round-to-nearest-even of w_hat.
R8  Matmul reference: the exact product of the bf16 operands, accumulated in
    fp64 (a library matmul is the step).  The fused kernel sums in another
    order, so the GEMM comparison is a tolerance, the codec comparison is
    bit-exact.
R9  8-bit maps (int8 "dynamic map", fp8 e4m3 codebook): not defined on the
    pages; an ascending 256-entry fp32 table passed in.
R10 8-bit packing: one index per byte, in element order.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

BLOCK = 64          # NF4 block (R3); "blocksize=64" in the #2034 reproducer
NESTED_BLOCK = 256  # nested 8-bit block (R5)

# R1: the 4-decimal NormalFloat-4 levels.  The pages name `code` as a
# QuantState field but never print its values.
_NF4_LEVELS_4DP = (
    -1.0, -0.6962, -0.5251, -0.3949, -0.2844, -0.1848, -0.0911, 0.0,
    0.0796, 0.1609, 0.2461, 0.3379, 0.4407, 0.5626, 0.7230, 1.0,
)


def nf4_code() -> np.ndarray:
    """The 16 NF4 levels as fp32 (R1)."""
    return np.array(_NF4_LEVELS_4DP, dtype=F32)


def uniform_nested_code() -> np.ndarray:
    """Symmetric uniform 8-bit table (2j - 255) / 255, j = 0..255, as fp32 (R6)."""
    j = np.arange(256, dtype=F64)
    return ((2.0 * j - 255.0) / 255.0).astype(F32)


def midpoints(code: np.ndarray) -> np.ndarray:
    """fp32 midpoints of adjacent table entries: fp32(code[j] + code[j+1]) / 2 (R4).

    The halving is exact in binary floating point, so only the sum rounds.
    """
    c = np.asarray(code, dtype=F32)
    s = (c[:-1] + c[1:]).astype(F32)
    return (s * F32(0.5)).astype(F32)


def nearest_index(t: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Number of midpoints strictly below each t (R4); result in 0..len(mids)."""
    t = np.asarray(t, dtype=F32)
    out = np.zeros(t.shape, dtype=np.int64)
    for m in mids:                      # one comparison per threshold
        out += (t > m)
    return out


def _blockwise_absmax(flat: np.ndarray, block: int) -> np.ndarray:
    """max |w| over consecutive blocks (last block may be partial); exact."""
    n = flat.shape[0]
    nb = -(-n // block)
    pad = nb * block - n
    a = np.abs(flat)
    if pad:
        a = np.concatenate([a, np.zeros(pad, dtype=a.dtype)])
    return a.reshape(nb, block).max(axis=1)


def _scale_to_unit(flat: np.ndarray, scale_per_block: np.ndarray, block: int) -> np.ndarray:
    """t = fp32(w / scale) per element, t = 0 where the block scale is 0 (R4)."""
    n = flat.shape[0]
    s = np.repeat(scale_per_block, block)[:n].astype(F32)
    t = np.zeros(n, dtype=F32)
    nz = s != 0
    t[nz] = (flat[nz].astype(F32) / s[nz]).astype(F32)
    return t


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two 4-bit indices per byte, element 2i in the high nibble (R2)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[0] % 2:
        raise ValueError("NF4 packing needs an even element count")
    return ((q[0::2] << 4) | q[1::2]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: returns the 4-bit indices in element order."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[0] * 2, dtype=np.uint8)
    q[0::2] = p >> 4
    q[1::2] = p & 0x0F
    return q


def absmax_mean_offset(absmax: np.ndarray) -> np.float32:
    """Mean of the fp32 absmax array in the fixed fp64 order of R5.

    Sequential fp64 sums inside consecutive chunks of 256 (the last may be
    partial), then a sequential fp64 sum of the chunk sums, an fp64 division
    by the count, and one rounding to fp32.  np.add.accumulate is a plain
    left-to-right running sum, so its last entry is the sequential sum.
    """
    a = np.asarray(absmax, dtype=F32).astype(F64)
    nb = a.shape[0]
    chunk_sums = []
    for start in range(0, nb, NESTED_BLOCK):
        part = a[start:start + NESTED_BLOCK]
        chunk_sums.append(np.add.accumulate(part)[-1])
    total = np.add.accumulate(np.array(chunk_sums, dtype=F64))[-1]
    return F32(total / F64(nb))


def quantize_nf4(w: np.ndarray, code: np.ndarray | None = None,
                 nested_code: np.ndarray | None = None, nested: bool = False) -> dict:
    """NF4 blockwise quantisation of W [N, K] (or any shape, flattened row-major).

    Steps (bitsandbytes #2034 "Minimal reproducer": quantize_4bit with
    blocksize 64, quant_type nf4, compress_statistics for the nested form):
      1. per block of 64: absmax = max |w|            (R3, exact)
      2. t = fp32(w / absmax), 0 for an all-zero block  (R4)
      3. q = #{j : t > mid[j]}                          (R4)
      4. pack two q per byte, high nibble first         (R2)
      5. nested only: offset, c = absmax - offset, per 256: s2 = max|c|,
         q2 = #{j : c/s2 > mid2[j]}                     (R5, R6)
    Input must be fp32 (a bf16 weight is widened exactly before the call).
    Returns dict(packed u8[n/2], absmax f32[nb] | u8[nb], nested_absmax
    f32[ng] | None, nested_offset f32 | None).
    """
    code = nf4_code() if code is None else np.asarray(code, dtype=F32)
    flat = np.ascontiguousarray(w, dtype=F32).reshape(-1)
    absmax = _blockwise_absmax(flat, BLOCK).astype(F32)
    t = _scale_to_unit(flat, absmax, BLOCK)
    q = nearest_index(t, midpoints(code))
    packed = pack_nibbles(q)
    if not nested:
        return dict(packed=packed, absmax=absmax, nested_absmax=None, nested_offset=None)

    ncode = uniform_nested_code() if nested_code is None else np.asarray(nested_code, dtype=F32)
    offset = absmax_mean_offset(absmax)
    c = (absmax - offset).astype(F32)
    s2 = _blockwise_absmax(c, NESTED_BLOCK).astype(F32)
    t2 = _scale_to_unit(c, s2, NESTED_BLOCK)
    q2 = nearest_index(t2, midpoints(ncode)).astype(np.uint8)
    return dict(packed=packed, absmax=q2, nested_absmax=s2, nested_offset=F32(offset))


def decode_absmax(absmax: np.ndarray, nested_absmax: np.ndarray | None = None,
                  nested_offset=None, nested_code: np.ndarray | None = None) -> np.ndarray:
    """Per-block fp32 scale (R7): plain fp32 absmax, or the nested decode
    fp32(fp32(nested_code[q2] * s2[b // 256]) + offset)."""
    if nested_absmax is None:
        return np.asarray(absmax, dtype=F32)
    ncode = uniform_nested_code() if nested_code is None else np.asarray(nested_code, dtype=F32)
    q2 = np.asarray(absmax, dtype=np.uint8).astype(np.int64)
    s2 = np.asarray(nested_absmax, dtype=F32)
    g = np.arange(q2.shape[0]) // NESTED_BLOCK
    prod = (ncode[q2] * s2[g]).astype(F32)
    return (prod + F32(nested_offset)).astype(F32)


def dequantize_nf4_f32(packed: np.ndarray, absmax: np.ndarray, nested_absmax=None,
                       nested_offset=None, code=None, nested_code=None,
                       n_elems: int | None = None) -> np.ndarray:
    """w_hat = fp32(code[q] * absmax_hat[block]) for every element (R7).

    bitsandbytes #2034 "Root cause": the backward multiplies by
    dequantize_4bit(B, state), the dense weight rebuilt from packed data and
    the QuantState fields.
    """
    code = nf4_code() if code is None else np.asarray(code, dtype=F32)
    q = unpack_nibbles(packed).astype(np.int64)
    if n_elems is not None:
        q = q[:n_elems]
    scale = decode_absmax(absmax, nested_absmax, nested_offset, nested_code)
    blk = np.arange(q.shape[0]) // BLOCK
    return (code[q] * scale[blk]).astype(F32)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit pattern of fp32 values by round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_rne_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bits of fp64 values by ONE round-to-nearest-even (normal range).

    The matmul output is returned in bf16, the dtype of the inputs (the
    F.linear convention kept by Soup #842, "Design sketch"), so the reference
    output is the exact product rounded once.  Rounding through fp32 first
    would round twice; here the fp64 significand is cut to bf16's 8 bits
    directly (bit 45 is the last kept bit), then the exact value is narrowed.
    """
    u = np.ascontiguousarray(x, dtype=F64).view(np.uint64)
    r = ((u + np.uint64(0x0FFFFFFFFFFF) + ((u >> np.uint64(45)) & np.uint64(1)))
         >> np.uint64(45)) << np.uint64(45)
    v = r.view(F64).astype(F32)                 # exact: at most 8 significant bits
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def dequantize_nf4_bf16_bits(packed, absmax, nested_absmax=None, nested_offset=None,
                             code=None, nested_code=None, n_elems=None) -> np.ndarray:
    """Dequantised weight in the compute dtype (bf16 bits), R7."""
    return bf16_rne_bits(dequantize_nf4_f32(packed, absmax, nested_absmax, nested_offset,
                                            code, nested_code, n_elems))


def _as_f64(bits_or_float: np.ndarray) -> np.ndarray:
    a = np.asarray(bits_or_float)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(F64)
    return a.astype(F64)


def matmul_fwd(x_bf16_bits: np.ndarray, w_bf16_bits: np.ndarray) -> np.ndarray:
    """y = x . W_hat^T in fp64 (R8).  x [M, K], W_hat [N, K] -> y [M, N].

    bitsandbytes #2034 "Minimal reproducer": matmul_4bit(h, w.t()) against
    the F.linear(h, w) control, W stored [out, in].
    """
    x = _as_f64(x_bf16_bits)
    w = _as_f64(w_bf16_bits)
    return x @ w.T


def matmul_bwd_input(gy_bf16_bits: np.ndarray, w_bf16_bits: np.ndarray) -> np.ndarray:
    """grad_x = grad_y . W_hat in fp64 (R8).  grad_y [M, N], W_hat [N, K].

    bitsandbytes #2034 "Root cause" (grad_A = grad_output @ dequantize_4bit(B))
    and Soup #842 "Design sketch" (the backward computes only grad_x).
    """
    gy = _as_f64(gy_bf16_bits)
    w = _as_f64(w_bf16_bits)
    return gy @ w


def grouped_matmul_fwd(x_bf16_bits: np.ndarray, offsets: np.ndarray,
                       w_stack_bf16_bits: np.ndarray) -> np.ndarray:
    """Per-expert forward on expert-sorted rows (Experts PR "Commit 2").

    x [T, K] sorted by expert; offsets [E+1]; W stack [E, N, K].
    Rows offsets[e]:offsets[e+1] use expert e's slice.
    """
    E, N, K = w_stack_bf16_bits.shape
    out = np.zeros((x_bf16_bits.shape[0], N), dtype=F64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = matmul_fwd(x_bf16_bits[lo:hi], w_stack_bf16_bits[e])
    return out


def grouped_matmul_bwd_input(gy_bf16_bits: np.ndarray, offsets: np.ndarray,
                             w_stack_bf16_bits: np.ndarray) -> np.ndarray:
    """Per-expert input gradient: grad_x[rows of e] = grad_y[rows of e] . W_hat_e."""
    E, N, K = w_stack_bf16_bits.shape
    out = np.zeros((gy_bf16_bits.shape[0], K), dtype=F64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = matmul_bwd_input(gy_bf16_bits[lo:hi], w_stack_bf16_bits[e])
    return out


# ---- 8-bit blockwise variants --------------------------------------------------
# bitsandbytes fork PR "Experts trainability ... ExpertsNbit", "Commit 1": its
# quant_type table lists 8-bit blockwise formats (int8 with a dynamic map, fp8
# e4m3 with its codebook) beside nf4 / fp4: one byte per weight, the same
# 64-element blocks and absmax (optionally double-quantised).  The pages do
# not define either 256-entry map, so (R9) the map is an explicit ascending
# 256-entry table passed in, exactly like the 16-entry NF4 code: the index is
# found by R4, one index per byte (R10), and the decode is R7 with this table.

def nearest_index_sorted(t: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Number of midpoints strictly below each t (R4), for midpoints in
    ascending order: the position of the first midpoint that is >= t, found
    by a sorted search (the library step; equal to the count of
    nearest_index)."""
    return np.searchsorted(np.asarray(mids, dtype=F32), np.asarray(t, dtype=F32), side="left")


def quantize_blockwise8(w: np.ndarray, code: np.ndarray, nested_code: np.ndarray | None = None,
                        nested: bool = False) -> dict:
    """8-bit blockwise quantisation of W (flattened row-major) with a
    256-entry ascending table: steps 1-3 and 5 of quantize_nf4, one index per
    byte in element order (R10).  Returns the same fields, packed u8[n]."""
    code = np.asarray(code, dtype=F32)
    if code.shape != (256,):
        raise ValueError("the 8-bit formats take a 256-entry table")
    flat = np.ascontiguousarray(w, dtype=F32).reshape(-1)
    absmax = _blockwise_absmax(flat, BLOCK).astype(F32)
    t = _scale_to_unit(flat, absmax, BLOCK)
    packed = nearest_index_sorted(t, midpoints(code)).astype(np.uint8)
    if not nested:
        return dict(packed=packed, absmax=absmax, nested_absmax=None, nested_offset=None)
    ncode = uniform_nested_code() if nested_code is None else np.asarray(nested_code, dtype=F32)
    offset = absmax_mean_offset(absmax)
    c = (absmax - offset).astype(F32)
    s2 = _blockwise_absmax(c, NESTED_BLOCK).astype(F32)
    t2 = _scale_to_unit(c, s2, NESTED_BLOCK)
    q2 = nearest_index(t2, midpoints(ncode)).astype(np.uint8)
    return dict(packed=packed, absmax=q2, nested_absmax=s2, nested_offset=F32(offset))


def dequantize_blockwise8_f32(packed: np.ndarray, absmax: np.ndarray, nested_absmax=None,
                              nested_offset=None, code=None, nested_code=None) -> np.ndarray:
    """w_hat = fp32(code[q] * absmax_hat[block]) with one byte per index (R7, R10)."""
    code = np.asarray(code, dtype=F32)
    q = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    scale = decode_absmax(absmax, nested_absmax, nested_offset, nested_code)
    blk = np.arange(q.shape[0]) // BLOCK
    return (code[q] * scale[blk]).astype(F32)


def dequantize_blockwise8_bf16_bits(packed, absmax, nested_absmax=None, nested_offset=None,
                                    code=None, nested_code=None) -> np.ndarray:
    """The 8-bit dequantised weight in the compute dtype (bf16 bits)."""
    return bf16_rne_bits(dequantize_blockwise8_f32(packed, absmax, nested_absmax, nested_offset,
                                                   code, nested_code))


# ---- storage accounting (bytes per format) ----------------------------------

def packed_bytes(n_elems: int, bits: int = 4) -> int:
    """Two 4-bit values per byte, or one 8-bit value (Experts PR "Commit 1" table)."""
    return n_elems // 2 if bits == 4 else n_elems


def absmax_count(n_elems: int) -> int:
    return -(-n_elems // BLOCK)


def nested_count(n_elems: int) -> int:
    return -(-absmax_count(n_elems) // NESTED_BLOCK)


def storage_bytes(n_elems: int, nested: bool, bits: int = 4) -> int:
    """Bytes of packed data + statistics for one quantised tensor."""
    nb = absmax_count(n_elems)
    if nested:
        return packed_bytes(n_elems, bits) + nb + 4 * nested_count(n_elems) + 4
    return packed_bytes(n_elems, bits) + 4 * nb
