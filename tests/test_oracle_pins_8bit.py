"""Pins of the oracle's 8-bit blockwise variants (bitsandbytes fork PR
"Experts trainability ... ExpertsNbit", "Commit 1" quant_type table: int8
blockwise and fp8 e4m3 beside nf4 / fp4, one byte per weight, the same
64-element blocks).  Each pin checks the oracle against something other than
itself: the tables against their definitions computed another way, the
quantiser against brute force and closed-form bounds, the sorted search
against the plain count, and the page's fidelity ordering."""

import numpy as np

import workloads as WL
from oracle import nf4_oracle as O

F32 = np.float32


def _e4m3_by_integers():
    """The e4m3 values as integer significands times powers of two:
    (8 [e > 0] + m) * 2^(max(e, 1) - 10) (bias 7, 3 mantissa bits)."""
    out = []
    for bits in range(256):
        e, m = (bits >> 3) & 15, bits & 7
        mag = np.ldexp(float(8 * (e > 0) + m), max(e, 1) - 10)
        out.append(-mag if bits & 0x80 else mag)
    return out


def test_fp8_table_matches_the_bit_fields():
    v = _e4m3_by_integers()
    assert max(v) == 480.0 and min(v) == -480.0
    assert sorted(abs(x) for x in v if x != 0)[0] == 2.0 ** -9          # smallest subnormal
    got = WL.fp8_e4m3_code_np()
    want = np.sort(np.array(v, dtype=np.float64)) / 480.0
    assert np.array_equal(got, want.astype(F32))                        # values (+-0 equal)
    assert np.signbit(got[127]) and not np.signbit(got[128])            # -0 before +0
    assert np.all(np.diff(got.astype(np.float64)) >= 0) and got[0] == -1 and got[-1] == 1
    # symmetric: entry 255 - j is minus entry j
    assert np.array_equal(got[::-1], -got)


def test_int8_table_closed_form():
    c = WL.int8_code_np()
    assert c.shape == (256,) and np.all(np.diff(c.astype(np.float64)) > 0)
    for j in (0, 1, 127, 128, 129, 255):
        assert c[j] == F32((j - 128) / 127)
    assert c[1] == -1 and c[128] == 0 and c[255] == 1


def test_sorted_search_equals_the_plain_count():
    g = np.random.default_rng(31)
    for code in (WL.int8_code_np(), WL.fp8_e4m3_code_np()):
        mids = O.midpoints(code)
        t = np.concatenate([g.uniform(-1, 1, 4000).astype(F32), mids, [F32(0), F32(-0.0), F32(1), F32(-1)]])
        assert np.array_equal(O.nearest_index_sorted(t, mids), O.nearest_index(t, mids))


def test_round_trip_on_table_values():
    """W built as fp32(code[q] * s) with a +-s element per block comes back
    exactly; repeated table values (+-0) come back as the lower index."""
    g = np.random.default_rng(32)
    for code in (WL.int8_code_np(), WL.fp8_e4m3_code_np()):
        nb = 150
        q = g.integers(1, 256, size=(nb, 64))
        q[:, 5] = g.choice([1 if code[0] < -1 else 0, 255], size=nb)
        s = (g.random(nb) * 3 + 0.01).astype(F32)
        w = (code[q] * s[:, None]).astype(F32)
        r = O.quantize_blockwise8(w.reshape(-1), code)
        assert np.array_equal(r["absmax"], s)
        got = r["packed"].reshape(nb, 64).astype(np.int64)
        lower = np.searchsorted(code, code[q], side="left")            # first index of that value
        assert np.array_equal(got, lower)
        d = O.dequantize_blockwise8_f32(r["packed"], r["absmax"], code=code)
        assert np.array_equal(d, w.reshape(-1))


def test_nearest_value_zero_and_bound():
    g = np.random.default_rng(33)
    w = (g.standard_normal(64 * 300) * 0.02).astype(F32)
    w[::13] = 0.0
    w[64 * 7:64 * 8] = 0.0                                              # an all-zero block
    for code in (WL.int8_code_np(), WL.fp8_e4m3_code_np()):
        r = O.quantize_blockwise8(w, code)
        q = r["packed"].astype(np.int64)
        t = (w.reshape(-1, 64) / np.where(r["absmax"] == 0, 1, r["absmax"])[:, None]).astype(F32)
        t = np.where(r["absmax"][:, None] == 0, F32(0), t).reshape(-1).astype(np.float64)
        c64 = code.astype(np.float64)
        best = np.abs(t[:, None] - c64[None, :]).min(axis=1)
        assert np.array_equal(np.abs(t - c64[q]), best)                 # a nearest value
        d = O.dequantize_blockwise8_f32(r["packed"], r["absmax"], code=code)
        assert np.all(d[w == 0] == 0)                                   # zeros stay zero
        half_gap = np.diff(c64[1:] if code[0] < -1 else c64).max() / 2
        assert np.all(np.abs(d - w).reshape(-1, 64) <= half_gap * r["absmax"][:, None] * (1 + 1e-6))
        # the block's largest magnitude comes back as +-absmax exactly
        blk = np.abs(w.reshape(-1, 64))
        i = blk.argmax(axis=1)
        rows = np.arange(blk.shape[0])
        nz = r["absmax"] > 0
        assert np.array_equal(np.abs(d.reshape(-1, 64)[rows, i])[nz], r["absmax"][nz])


def test_fidelity_ordering_int8_fp8_nf4():
    """The Experts PR ("Commit 1" / its fidelity test) ranks the formats by
    reconstruction error: int8 blockwise more than 4x below nf4 in mean
    |w - w_hat|; fp8 e4m3 also below nf4."""
    g = np.random.default_rng(34)
    w = (g.standard_normal(64 * 4000) * 0.02).astype(F32)
    r4 = O.quantize_nf4(w)
    e4 = np.abs(O.dequantize_nf4_f32(r4["packed"], r4["absmax"]) - w).mean()
    e = {}
    for name, code in (("int8", WL.int8_code_np()), ("fp8", WL.fp8_e4m3_code_np())):
        r = O.quantize_blockwise8(w, code)
        e[name] = np.abs(O.dequantize_blockwise8_f32(r["packed"], r["absmax"], code=code) - w).mean()
    assert 4 * e["int8"] < e4
    assert e["fp8"] < e4


def test_nested_8bit_statistics_match_the_4bit_path():
    """The block statistics do not depend on the element format: the nested
    fields of the 8-bit quantiser equal those of the NF4 quantiser."""
    g = np.random.default_rng(35)
    w = (g.standard_normal(64 * 256 * 3) * 0.02).astype(F32)
    r8 = O.quantize_blockwise8(w, WL.int8_code_np(), nested=True)
    r4 = O.quantize_nf4(w, nested=True)
    for k in ("absmax", "nested_absmax"):
        assert np.array_equal(r8[k], r4[k])
    assert r8["nested_offset"] == r4["nested_offset"]
    assert O.storage_bytes(w.size, True, bits=8) == w.size + w.size // 64 + 4 * 3 + 4
