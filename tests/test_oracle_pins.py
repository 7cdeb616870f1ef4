"""Pins of the CPU oracle against facts other than itself (no GPU needed).

Each test ties one oracle step to a closed form, a brute-force computation,
an invariant of the encoding, or a figure printed on the pages, chosen so a
plausible mistake in the oracle (a dropped term, a wrong sign, a swapped
nibble, a transposed operand, a different tie rule) fails one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import nf4_oracle as O
import workloads as WL

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- code tables -------------------------------------------------------------

def test_code_table_matches_normalfloat_construction():
    """The 16 levels are the normalised N(0,1) quantiles of the NormalFloat
    construction (QLoRA): 8 positive quantiles on [1-d, 1/2), 7 negative ones
    mirrored, an exact zero, d = (1/32 + 1/30)/2, scaled to max 1.  The stored
    4-decimal values agree within half a unit of the 4th decimal (+1e-7 for the
    construction's own float evaluation)."""
    from scipy.stats import norm
    d = 0.5 * (1 / 32 + 1 / 30)
    pos = norm.ppf(np.linspace(1 - d, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(1 - d, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, neg, [0.0]]))
    v = v / np.abs(v).max()
    code = O.nf4_code().astype(np.float64)
    assert np.all(np.diff(code) > 0)
    assert np.abs(v - code).max() <= 5e-5 + 1e-7


def test_input_tables_are_the_oracle_defaults():
    """The tables every GPU call receives (inputs) equal the oracle's defaults."""
    assert np.array_equal(WL.nf4_code_np(), O.nf4_code())
    assert np.array_equal(WL.nested_code_np(), O.uniform_nested_code())


def test_nested_table_closed_form():
    c = O.uniform_nested_code().astype(np.float64)
    assert c.shape == (256,)
    assert c[0] == -1.0 and c[-1] == 1.0
    assert np.all(c == -c[::-1])                         # symmetric
    assert np.allclose(np.diff(c), 2 / 255, rtol=0, atol=1e-7)
    assert np.all(np.diff(c) > 0)


# --- NF4 quantise / dequantise ---------------------------------------------

def test_pack_order_closed_form():
    """w[k] = 2 * code[k % 16] has absmax 2 and t = code[q] exactly, so the
    indices run 0..15 and, high nibble first, the bytes are 0x01 0x23 ... 0xEF."""
    code = O.nf4_code()
    w = np.tile((code * F32(2.0)).astype(F32), 8).reshape(2, 64)
    r = O.quantize_nf4(w)
    assert np.all(r["absmax"] == F32(2.0))
    assert list(r["packed"][:8]) == [0x01, 0x23, 0x45, 0x67, 0x89, 0xAB, 0xCD, 0xEF]
    assert np.array_equal(O.dequantize_nf4_f32(r["packed"], r["absmax"]), w.reshape(-1))


def test_round_trip_on_code_values():
    """A weight built as fp32(code[q] * s) with one +-s element per block
    round-trips exactly: indices and values."""
    g = np.random.default_rng(11)
    code = O.nf4_code()
    nb = 300
    q = g.integers(0, 16, size=(nb, 64))
    q[:, 5] = g.choice([0, 15], size=nb)             # guarantees max |.| = s
    s = (g.random(nb) * 3 + 0.01).astype(F32)
    w = (code[q] * s[:, None]).astype(F32)
    r = O.quantize_nf4(w.reshape(-1))
    assert np.array_equal(r["absmax"], s)
    assert np.array_equal(O.unpack_nibbles(r["packed"]).reshape(nb, 64), q)
    assert np.array_equal(O.dequantize_nf4_f32(r["packed"], r["absmax"]), w.reshape(-1))


def test_zero_preserved_and_zero_block():
    g = np.random.default_rng(1)
    w = (g.standard_normal(64 * 20) * 0.02).astype(F32)
    w[::7] = 0.0
    w[64:128] = 0.0                                   # one all-zero block
    r = O.quantize_nf4(w)
    d = O.dequantize_nf4_f32(r["packed"], r["absmax"])
    assert np.all(d[w == 0] == 0.0)
    assert r["absmax"][1] == 0.0
    assert np.all(O.unpack_nibbles(r["packed"])[64:128] == 7)


def test_block_max_element_reproduces_absmax():
    g = np.random.default_rng(2)
    w = (g.standard_normal((40, 64)) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    d = O.dequantize_nf4_f32(r["packed"], r["absmax"]).reshape(40, 64)
    i = np.abs(w).argmax(axis=1)
    rows = np.arange(40)
    assert np.array_equal(d[rows, i], np.sign(w[rows, i]) * np.abs(w[rows, i]))


def test_index_is_brute_force_nearest_code():
    g = np.random.default_rng(3)
    w = (g.standard_normal(64 * 500) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    code = O.nf4_code().astype(np.float64)
    t = (w.reshape(-1, 64) / r["absmax"][:, None]).astype(F32).astype(np.float64).reshape(-1)
    dist = np.abs(t[:, None] - code[None, :])
    best = dist.argmin(axis=1)
    srt = np.sort(dist, axis=1)
    assert np.all(srt[:, 1] - srt[:, 0] > 1e-6)       # no near-ties in this draw
    assert np.array_equal(O.unpack_nibbles(r["packed"]), best)


def test_exact_midpoint_goes_to_lower_code():
    """With absmax 1, w = mid[j] gives t = mid[j] exactly; strict '>' sends it
    to index j (the lower neighbour)."""
    mids = O.midpoints(O.nf4_code())
    w = np.zeros(64, dtype=F32)
    w[0] = 1.0
    w[1:16] = mids
    q = O.unpack_nibbles(O.quantize_nf4(w)["packed"])
    assert q[0] == 15
    assert list(q[1:16]) == list(range(15))


def test_error_bound_and_monotone():
    g = np.random.default_rng(4)
    w = (g.standard_normal((64, 64)) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    d = O.dequantize_nf4_f32(r["packed"], r["absmax"]).reshape(64, 64)
    half_gap = np.diff(O.nf4_code().astype(np.float64)).max() / 2   # (1 - 0.6962)/2
    assert abs(half_gap - 0.1519) < 1e-6
    bound = half_gap * r["absmax"][:, None] * (1 + 1e-6) + 1e-12
    assert np.all(np.abs(d - w) <= bound)
    for b in range(64):                               # monotone inside a block
        o = np.argsort(w[b], kind="stable")
        assert np.all(np.diff(d[b][o]) >= 0)


def test_bf16_rne_special_cases():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -1.0 - 2 ** -8, 0.0, -0.0, 3.0e38], dtype=F32)
    b = O.bf16_rne_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 tie -> up to 1 + 2^-6;
    # just above the tie -> up; sign symmetric; zeros keep their sign.
    assert list(b[:7]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x0000, 0x8000]
    assert np.array_equal(O.bf16_bits_to_f32(b)[:2], np.array([1.0, 1.0], F32))


def test_bf16_single_rounding_from_f64():
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie: one rounding goes up, while
    # rounding through fp32 first lands exactly on the tie and goes to even.
    v = np.array([1.0 + 2 ** -8 + 2 ** -30, -(1.0 + 2 ** -8 + 2 ** -30)])
    assert list(O.bf16_rne_bits_from_f64(v)) == [0x3F81, 0xBF81]
    assert list(O.bf16_rne_bits(v.astype(F32))) == [0x3F80, 0xBF80]
    # on values exactly representable in fp32 both routes agree
    g = np.random.default_rng(12)
    x = (g.standard_normal(20000) * 10.0 ** g.integers(-3, 3, 20000)).astype(F32)
    assert np.array_equal(O.bf16_rne_bits_from_f64(x.astype(np.float64)), O.bf16_rne_bits(x))
    # and the result is the nearest bf16 value (brute force over neighbours)
    y = g.standard_normal(5000)
    b = O.bf16_rne_bits_from_f64(y)
    val = O.bf16_bits_to_f32(b).astype(np.float64)
    for d in (-1, 1):
        nb = O.bf16_bits_to_f32((b.astype(np.int32) + d).astype(np.uint16)).astype(np.float64)
        assert np.all(np.abs(y - val) <= np.abs(y - nb))


# --- nested statistics ---------------------------------------------------------

def test_offset_is_the_mean_in_fixed_order():
    g = np.random.default_rng(5)
    a = (np.abs(g.standard_normal(256 * 5 + 77)) * 0.05).astype(F32)
    off = O.absmax_mean_offset(a)
    exact = math.fsum(float(v) for v in a) / len(a)
    assert abs(float(off) - exact) <= np.spacing(F32(exact))
    # the fixed order, spelled out as plain Python loops in fp64
    chunks = []
    for s in range(0, len(a), 256):
        acc = 0.0
        for v in a[s:s + 256]:
            acc += float(v)
        chunks.append(acc)
    tot = 0.0
    for c in chunks:
        tot += c
    assert off == F32(tot / len(a))


def test_nested_decode_bounds_and_endpoints():
    g = np.random.default_rng(6)
    w = (g.standard_normal((64, 1024)) * 0.02).astype(F32)
    plain = O.quantize_nf4(w)
    nest = O.quantize_nf4(w, nested=True)
    assert nest["absmax"].dtype == np.uint8
    a = plain["absmax"]
    ah = O.decode_absmax(nest["absmax"], nest["nested_absmax"], nest["nested_offset"])
    s2 = np.repeat(nest["nested_absmax"], 256)[:a.shape[0]]
    off = nest["nested_offset"]
    tol = s2.astype(np.float64) / 255 * (1 + 1e-5) + 4 * np.spacing(np.abs(a) + np.abs(off))
    assert np.all(np.abs(ah.astype(np.float64) - a) <= tol)
    c = (a - off).astype(F32)
    for gi in range(nest["nested_absmax"].shape[0]):
        seg = slice(gi * 256, (gi + 1) * 256)
        j = np.abs(c[seg]).argmax()
        sgn = np.sign(c[seg][j])
        assert ah[seg][j] == F32(sgn * nest["nested_absmax"][gi] + off)


def test_nested_dequant_uses_decoded_scale():
    g = np.random.default_rng(7)
    w = (g.standard_normal((8, 512)) * 0.02).astype(F32)
    nest = O.quantize_nf4(w, nested=True)
    ah = O.decode_absmax(nest["absmax"], nest["nested_absmax"], nest["nested_offset"])
    q = O.unpack_nibbles(nest["packed"]).astype(np.int64)
    manual = np.array([F32(O.nf4_code()[q[i]] * ah[i // 64]) for i in range(q.shape[0])], F32)
    d = O.dequantize_nf4_f32(nest["packed"], nest["absmax"], nest["nested_absmax"],
                             nest["nested_offset"])
    assert np.array_equal(d, manual)


# --- matmul reference ----------------------------------------------------------

def _brute_fwd(x, w):
    M, K = x.shape
    N = w.shape[0]
    y = np.zeros((M, N))
    for m, n in itertools.product(range(M), range(N)):
        acc = 0.0
        for k in range(K):
            acc += float(x[m, k]) * float(w[n, k])
        y[m, n] = acc
    return y


def _brute_bwd(gy, w):
    M, N = gy.shape
    K = w.shape[1]
    gx = np.zeros((M, K))
    for m, k in itertools.product(range(M), range(K)):
        acc = 0.0
        for n in range(N):
            acc += float(gy[m, n]) * float(w[n, k])
        gx[m, k] = acc
    return gx


@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (7, 2, 128), (1, 9, 64)])
def test_matmul_brute_force(M, N, K):
    g = np.random.default_rng(M * 100 + N)
    w = (g.standard_normal((N, K)) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    wb = O.dequantize_nf4_bf16_bits(r["packed"], r["absmax"]).reshape(N, K)
    x = O.bf16_rne_bits(g.standard_normal((M, K)).astype(F32))
    gy = O.bf16_rne_bits(g.standard_normal((M, N)).astype(F32))
    xf, wf, gyf = (O.bf16_bits_to_f32(v) for v in (x, wb, gy))
    y = O.matmul_fwd(x, wb)
    gx = O.matmul_bwd_input(gy, wb)
    assert y.shape == (M, N) and gx.shape == (M, K)
    np.testing.assert_allclose(y, _brute_fwd(xf, wf), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gx, _brute_bwd(gyf, wf), rtol=1e-12, atol=1e-12)


def test_identity_and_permutation_probes():
    g = np.random.default_rng(8)
    N, K = 64, 128
    w = (g.standard_normal((N, K)) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    wb = O.dequantize_nf4_bf16_bits(r["packed"], r["absmax"]).reshape(N, K)
    wf = O.bf16_bits_to_f32(wb).astype(np.float64)
    eye_k = O.bf16_rne_bits(np.eye(K, dtype=F32))
    eye_n = O.bf16_rne_bits(np.eye(N, dtype=F32))
    assert np.array_equal(O.matmul_fwd(eye_k, wb), wf.T)
    assert np.array_equal(O.matmul_bwd_input(eye_n, wb), wf)
    p = g.permutation(K)
    perm_x = O.bf16_rne_bits(np.eye(K, dtype=F32)[p])
    assert np.array_equal(O.matmul_fwd(perm_x, wb), wf.T[p])


def test_grouped_matches_per_expert_loops():
    g = np.random.default_rng(9)
    E, N, K = 5, 16, 64
    w = (g.standard_normal((E, N, K)) * 0.02).astype(F32)
    r = O.quantize_nf4(w)
    wb = O.dequantize_nf4_bf16_bits(r["packed"], r["absmax"]).reshape(E, N, K)
    counts = np.array([3, 0, 5, 1, 0])                   # includes empty experts
    offsets = np.concatenate([[0], np.cumsum(counts)])
    T = offsets[-1]
    x = O.bf16_rne_bits(g.standard_normal((T, K)).astype(F32))
    gy = O.bf16_rne_bits(g.standard_normal((T, N)).astype(F32))
    y = O.grouped_matmul_fwd(x, offsets, wb)
    gx = O.grouped_matmul_bwd_input(gy, offsets, wb)
    for e in range(E):
        for row in range(offsets[e], offsets[e + 1]):
            xf = O.bf16_bits_to_f32(x[row:row + 1])
            gyf = O.bf16_bits_to_f32(gy[row:row + 1])
            wf = O.bf16_bits_to_f32(wb[e])
            np.testing.assert_allclose(y[row], _brute_fwd(xf, wf)[0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(gx[row], _brute_bwd(gyf, wf)[0], rtol=1e-12, atol=1e-12)


# --- storage accounting against figures the pages print -------------------------

def _golden():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


def _layer_elems(projs):
    return [p.N * p.K for p in projs]


def test_llama_dequant_bytes_and_calls():
    G = _golden()
    elems = sum(_layer_elems(WL.LLAMA_8B))
    assert elems == 218_103_808
    mb = elems * 2 / 1e6                                 # dense bf16 written per visit
    assert abs(mb - G["dequant_vram_per_layer_visit_MB"]["value"]) / mb < 0.005
    assert len(WL.LLAMA_8B) * WL.LLAMA_LAYERS * 2 == G["dequant_calls_per_step"]["value"]


def test_bf16_vs_nested_nf4_ratio():
    G = _golden()
    elems = _layer_elems(WL.LLAMA_8B)
    nf4 = sum(O.storage_bytes(e, nested=True) for e in elems)
    ratio = sum(elems) * 2 / nf4
    assert abs(ratio - 3.877) < 0.005
    assert round(ratio, 1) == G["bf16_over_nf4_bytes_per_layer"]["value"]


def test_qwen_layer_bytes_match_repair_cost():
    G = _golden()
    elems = _layer_elems(WL.QWEN_32B)
    layer = sum(O.storage_bytes(e, nested=True) for e in elems)
    assert layer == 251_531_548
    mib = layer / 2 ** 20
    page = G["repair_extra_MiB"]["value"] / G["repair_extra_layer_equivalents"]["value"]
    assert abs(mib - page) / page < 0.005
    d = G["dealias_peak_MiB"]
    assert abs(64 * mib - (d["after"] - d["before"])) / (d["after"] - d["before"]) < 0.02


def test_olmoe_saved_dense_weights():
    G = _golden()
    dense = WL.OLMOE_E * 3 * WL.OLMOE_INTER * WL.OLMOE_HIDDEN * 2 / 1e6
    page = G["olmoe_saved_dense_weights_MB_per_layer"]["value"]
    assert abs(dense - page) / page < 0.03


def test_unnested_storage_formula():
    assert O.storage_bytes(128 * 256, nested=False) == 128 * 256 // 2 + 4 * 512
    assert O.absmax_count(65) == 2 and O.nested_count(64 * 257) == 2


# --- fp4: the same codec with another 16-entry table (Experts PR, "Commit 1"
# table: nf4 / fp4 share the 4-bit packed path) ---------------------------------

def _e2m1_values():
    """The 16 values of a float with 1 sign, 2 exponent (bias 1) and 1
    mantissa bit, decoded from the bit fields (exponent 0 is subnormal)."""
    out = []
    for bits in range(16):
        sign = -1.0 if bits & 8 else 1.0
        e, m = (bits >> 1) & 3, bits & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
        out.append(sign * mag)
    return out


def test_fp4_table_is_e2m1_over_its_max():
    import math
    v = sorted(_e2m1_values(), key=lambda x: (x, math.copysign(1.0, x) > 0))
    want = (np.array(v, dtype=np.float64) / max(abs(x) for x in v)).astype(F32)
    got = WL.fp4_code_np()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))   # -0 before +0
    assert np.signbit(got[7]) and not np.signbit(got[8])
    assert np.all(np.diff(got.astype(np.float64)) >= 0)


def test_fp4_round_trip_on_code_values():
    """fp32(code[q] * s) with a +-s element per block comes back exactly as a
    value; the +0 entry comes back as index 7 (-0), equal in value."""
    g = np.random.default_rng(21)
    code = WL.fp4_code_np()
    nb = 200
    q = g.integers(0, 16, size=(nb, 64))
    q[:, 3] = g.choice([0, 15], size=nb)
    s = (g.random(nb) * 3 + 0.01).astype(F32)
    w = (code[q] * s[:, None]).astype(F32)
    r = O.quantize_nf4(w.reshape(-1), code=code)
    assert np.array_equal(r["absmax"], s)
    got_q = O.unpack_nibbles(r["packed"]).reshape(nb, 64)
    assert np.array_equal(got_q, np.where(q == 8, 7, q))
    d = O.dequantize_nf4_f32(r["packed"], r["absmax"], code=code)
    assert np.array_equal(d, w.reshape(-1))                            # -0 == +0 as values


def test_fp4_nearest_value_brute_force_and_bound():
    g = np.random.default_rng(22)
    code = WL.fp4_code_np()
    w = (g.standard_normal(64 * 400) * 0.02).astype(F32)
    w[::11] = 0.0
    r = O.quantize_nf4(w, code=code)
    q = O.unpack_nibbles(r["packed"])
    t = (w.reshape(-1, 64) / r["absmax"][:, None]).astype(F32).astype(np.float64).reshape(-1)
    c64 = code.astype(np.float64)
    best = np.abs(t[:, None] - c64[None, :]).min(axis=1)
    assert np.array_equal(np.abs(t - c64[q]), best)                   # a nearest value
    # sign kept: t <= 0 maps to a non-positive code (-0 included), t > 0 to a non-negative one
    assert np.all(np.signbit(code[q][t <= 0])) and not np.any(np.signbit(code[q][t > 0]))
    d = O.dequantize_nf4_f32(r["packed"], r["absmax"], code=code).reshape(-1, 64)
    half_gap = np.diff(c64).max() / 2                                   # (1 - 2/3) / 2
    assert abs(half_gap - 1 / 6) < 1e-7
    assert np.all(np.abs(d - w.reshape(-1, 64)) <= half_gap * r["absmax"][:, None] * (1 + 1e-6))


def test_nf4_beats_fp4_on_normal_weights():
    """On N(0, s) weights the NormalFloat levels reconstruct with a lower
    mean-abs error than the float levels (the reason NF4 is the default)."""
    g = np.random.default_rng(23)
    w = (g.standard_normal(64 * 2000) * 0.02).astype(F32)
    err = {}
    for name, code in (("nf4", O.nf4_code()), ("fp4", WL.fp4_code_np())):
        r = O.quantize_nf4(w, code=code)
        err[name] = np.abs(O.dequantize_nf4_f32(r["packed"], r["absmax"], code=code) - w).mean()
    assert err["nf4"] < err["fp4"]
