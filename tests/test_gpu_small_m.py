"""GPU parity of the weight-streaming forward (M <= 32) against the oracle.

* the path counters show the streaming kernel ran (and the split reduction
  when the contraction is chunked);
* permutation probes: rows of x are unit vectors, so y[m] = W_hat[:, p(m)]
  bit for bit -- the expansion order and the permuted staging of x agree;
* seeded tolerance checks at M = 1 .. 32 over ragged N, contraction lengths
  that end inside a step, plain and nested statistics;
* full-size Llama-3.1-8B decode shapes (M = 1, 8, 32) in the launch
  configuration the benchmark times, checked on sampled output columns;
* bitwise run-to-run determinism, and agreement with the tiled kernel
  (NF4_SMALL_M=0) through the same oracle.
"""

import os

import numpy as np
import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from oracle import nf4_oracle as O

from gpu_util import DEV, abs_bits, assert_close, bits_of, ref_bits, upload

pytestmark = pytest.mark.gpu


def _setup(M, N, K, nested, seed):
    w = WL.weight_f32(N, K, WL.W_DECODE, 2000 + seed)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    wb = ref_bits(ref, (N, K))
    x = WL.x_bf16(M, K, WL.W_DECODE, 2000 + seed)
    return wq, wb, x


@pytest.mark.parametrize("N,K", [(200, 576), (208, 512)])   # ragged (32-row kernel); whole steps and row groups
@pytest.mark.parametrize("M", [1, 16, 17, 32])
@pytest.mark.parametrize("nested", [False, True])
def test_permutation_probe_small_m(M, nested, N, K):
    w = WL.weight_f32(N, K, WL.W_DECODE, 40 + M)
    ref = O.quantize_nf4(w, nested=nested)
    wq = upload(ref, N, K, nested)
    wb = ref_bits(ref, (N, K))
    p = np.random.default_rng(M).integers(0, K, size=M)
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[np.arange(M), p] = 1.0
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    torch.cuda.synchronize()
    assert api.nf4_path_counts()["fwd_small_m"] == 1
    assert np.array_equal(bits_of(y), wb.T[p])


SMALL = [
    (1, 64, 64), (1, 1000, 4160), (2, 136, 320), (7, 520, 1088), (16, 257, 2048),
    (17, 96, 448), (24, 1024, 1024), (32, 130, 4096), (32, 2048, 192),
]


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_m_vs_oracle(M, N, K, nested):
    wq, wb, x = _setup(M, N, K, nested, M + N + K)
    xb = WL.bf16_bits(x)
    api.nf4_reset_path_counts()
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    torch.cuda.synchronize()
    c = api.nf4_path_counts()
    assert c["fwd_small_m"] == 1 and c["fwd_tiled"] == 0
    splits_expected = api.nf4_workspace_bytes(1, M, N, K) > 0
    assert (c["splitk_reduce"] == 1) == splits_expected
    assert_close(y, O.matmul_fwd(xb, wb), f"y {M}x{N}x{K}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)


def test_small_m_matches_tiled_and_repeats():
    M, N, K = 8, 1536, 3072
    wq, wb, x = _setup(M, N, K, True, 5)
    xd = x.to(DEV)
    y0 = api.nf4_matmul_fwd(xd, wq).clone()
    for _ in range(3):
        assert torch.equal(api.nf4_matmul_fwd(xd, wq).view(torch.int16), y0.view(torch.int16))
    old = os.environ.get("NF4_SMALL_M")
    os.environ["NF4_SMALL_M"] = "0"
    try:
        api.nf4_reset_path_counts()
        yt = api.nf4_matmul_fwd(xd, wq)
        torch.cuda.synchronize()
        assert api.nf4_path_counts()["fwd_tiled"] == 1
    finally:
        if old is None:
            del os.environ["NF4_SMALL_M"]
        else:
            os.environ["NF4_SMALL_M"] = old
    want = O.matmul_fwd(WL.bf16_bits(x), wb)
    assert_close(y0, want, "streaming")
    assert_close(yt, want, "tiled")


@pytest.mark.parametrize("M", list(WL.DECODE_MS))
@pytest.mark.parametrize("idx", [0, 1, 4, 6])    # q/o (4096), k/v (N = 1024), gate/up (14336), down (K = 14336)
def test_llama_decode_shapes(M, idx):
    p = WL.LLAMA_8B[idx]
    w = WL.weight_f32(p.N, p.K, WL.W_LLAMA, 0, idx)
    ref = O.quantize_nf4(w, nested=True)
    del w
    wq = upload(ref, p.N, p.K, True)
    x = WL.x_bf16(M, p.K, WL.W_LLAMA, 0)
    xb = WL.bf16_bits(x)
    y = api.nf4_matmul_fwd(x.to(DEV), wq)
    # sampled output columns: the oracle dequantises only those rows of W
    cols = np.sort(np.random.default_rng(idx * 100 + M).choice(p.N, size=96, replace=False))
    cols[0], cols[-1] = 0, p.N - 1
    wb = ref_bits(ref, (p.N, p.K))[cols]
    assert_close(y[:, torch.from_numpy(cols).to(DEV)], O.matmul_fwd(xb, wb), f"{p.name} M={M}",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb)), p.K)
    y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not bitwise repeatable"


@pytest.mark.parametrize("M,rw,mp32", [
    (1, None, None), (5, 1, None), (5, 2, None), (5, 4, None), (16, 4, None),   # 16-row groups
    (17, 1, "0"), (20, 2, "0"), (24, 4, "0"),                                  # two halves of x
    (17, None, "1"), (32, None, None)])                                         # 32-row groups
@pytest.mark.parametrize("kw", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("z", [1, 3])
def test_small_m_slices_and_chunks(M, rw, mp32, kw, z):
    """Every (row-group size, row groups, contraction slices, chunks) instance
    of the streaming kernels through the documented overrides: slices past a
    short contraction hold no steps, and with four row groups the last
    workgroup holds a row group past N.  (N and K are whole 16-row groups and
    256-column steps, the shapes the 16-row kernel takes; chunks of the
    32-row kernel end inside its steps.)"""
    N, K = 304, 1536
    nested = (kw + z) % 2 == 0
    wq, wb, x = _setup(M, N, K, nested, 7 * kw + z + M)
    xb = WL.bf16_bits(x)
    old = {k: os.environ.get(k) for k in ("NF4_GEMV_KW", "NF4_GEMV_Z", "NF4_GEMV_RW", "NF4_GEMV_MP32")}
    os.environ["NF4_GEMV_KW"], os.environ["NF4_GEMV_Z"] = str(kw), str(z)
    if rw is not None:
        os.environ["NF4_GEMV_RW"] = str(rw)
    if mp32 is not None:
        os.environ["NF4_GEMV_MP32"] = mp32
    try:
        ws_bytes = api.nf4_workspace_bytes(1, M, N, K)
        api.nf4_reset_path_counts()
        y = api.nf4_matmul_fwd(x.to(DEV), wq)
        y2 = api.nf4_matmul_fwd(x.to(DEV), wq)
        torch.cuda.synchronize()
        c = api.nf4_path_counts()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert c["fwd_small_m"] == 2
    # chunks come from the override or from the x chunk's LDS budget
    assert (c["splitk_reduce"] == 2) == (ws_bytes > 0)
    assert ws_bytes > 0 or z == 1
    if not torch.equal(y.view(torch.int16), y2.view(torch.int16)):
        ref = O.quantize_nf4(WL.weight_f32(N, K, WL.W_DECODE, 2000 + 7 * kw + z + M), nested=nested)
        for name in ("packed", "absmax"):
            t = getattr(wq, name)
            host = np.asarray(ref[name]).reshape(-1)
            a = t.cpu().numpy().reshape(-1)
            b = t.clone().cpu().numpy().reshape(-1)
            c = (t.view(torch.uint8).to(torch.int32) + 0).to(torch.uint8).cpu().numpy().reshape(-1) if name == "packed" else b
            print("DIAG", name, "copy==ref", bool(np.array_equal(a.view(np.uint8), host.view(np.uint8))),
                  "clone==ref", bool(np.array_equal(b.view(np.uint8), host.view(np.uint8))),
                  "kernelread==ref", bool(np.array_equal(c.view(np.uint8), host.view(np.uint8))),
                  "first bad clone byte", int(np.argmax(b.view(np.uint8) != host.view(np.uint8))) if not np.array_equal(b.view(np.uint8), host.view(np.uint8)) else -1,
                  "nbytes", host.view(np.uint8).size, "ptr", hex(t.data_ptr()), flush=True)
        xd1 = x.to(DEV)
        print("DIAG x copy==", bool(np.array_equal(xd1.cpu().view(torch.int16).numpy(), x.view(torch.int16).numpy())),
              "x clone==", bool(np.array_equal(xd1.clone().cpu().view(torch.int16).numpy(), x.view(torch.int16).numpy())), flush=True)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not bitwise repeatable"
    assert_close(y, O.matmul_fwd(xb, wb), f"y M={M} rw={rw} mp32={mp32} kw={kw} z={z}",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("z", [1, 3])
@pytest.mark.parametrize("M", [5, 24])
def test_small_m_four_row_groups(M, z, nested):
    """Four row groups per workgroup (two slices), N a multiple of 64 so that
    every workgroup's row groups are whole, with and without chunks: two
    calls bitwise equal and matching the oracle."""
    N, K = 320, 1536
    wq, wb, x = _setup(M, N, K, nested, 11 * M + z)
    keys = ("NF4_GEMV_KW", "NF4_GEMV_Z", "NF4_GEMV_RW", "NF4_GEMV_MP32")
    old = {k: os.environ.get(k) for k in keys}
    os.environ.update({"NF4_GEMV_KW": "2", "NF4_GEMV_Z": str(z), "NF4_GEMV_RW": "4", "NF4_GEMV_MP32": "0"})
    try:
        xd = x.to(DEV)
        y = api.nf4_matmul_fwd(xd, wq)
        y2 = api.nf4_matmul_fwd(xd, wq)
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not bitwise repeatable"
    xb = WL.bf16_bits(x)
    assert_close(y, O.matmul_fwd(xb, wb), f"y M={M} z={z}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)


@pytest.mark.parametrize("kw", ["2", "4"])
@pytest.mark.parametrize("N,K", [(144, 256), (144, 512), (160, 768)])
def test_small_m_one_step_waves_repeat(N, K, kw):
    """Contraction slices of one step each (and empty ones), nested scales:
    thirty calls in a row are bitwise equal and match the oracle.  (Covers the
    stale reads a wave once got when a repeat copy of the lines it waited for
    was still in flight.)"""
    M = 2
    wq, wb, x = _setup(M, N, K, True, M + N + K)
    want = O.matmul_fwd(WL.bf16_bits(x), wb)
    old = os.environ.get("NF4_GEMV_KW")
    os.environ["NF4_GEMV_KW"] = kw
    try:
        xd = x.to(DEV)
        ys = [api.nf4_matmul_fwd(xd, wq) for _ in range(30)]
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("NF4_GEMV_KW", None)
        else:
            os.environ["NF4_GEMV_KW"] = old
    for i, y in enumerate(ys):
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), f"call {i} differs"
    assert_close(ys[0], want, f"y {M}x{N}x{K} kw={kw}")


@pytest.mark.parametrize("M,N,K", [(1, 1008, 4096), (1, 272, 1024), (8, 1008, 4096), (3, 528, 8192)])
def test_small_m_nested_first_steps_repeat(M, N, K):
    """Nested statistics, many short waves whose first steps start right after
    the prologue: a hundred calls in a row are bitwise equal and the first
    matches the oracle.  (Covers the stale nested scale a wave read at its
    first step while the copy of the next step's scale, from the same address,
    was still in flight.)"""
    wq, wb, x = _setup(M, N, K, True, 31 * M + N + K)
    xd = x.to(DEV)
    ys = [api.nf4_matmul_fwd(xd, wq) for _ in range(100)]
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), f"call {i} differs"
    xb = WL.bf16_bits(x)
    assert_close(ys[0], O.matmul_fwd(xb, wb), f"y {M}x{N}x{K}", O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)


@pytest.mark.parametrize("nested", [False, True])
@pytest.mark.parametrize("rw,kw", [("4", "2"), ("1", "4"), ("2", "2")])
@pytest.mark.parametrize("M,N,K", [(5, 300, 1600), (1, 136, 1088), (8, 264, 320), (5, 304, 1536)])
def test_small_m_ragged_rows_repeat(M, N, K, rw, kw, nested):
    """Ragged shapes (K not a multiple of 256, N not of 16: the 32-row kernel
    takes them) and whole-step shapes with a row group past N in the last
    workgroup (the 16-row kernel), several contraction slices and row groups
    per workgroup: fifty calls in a row are bitwise equal and the first
    matches the oracle.  (The 16-row kernel once copied, on a ragged last
    step, the head of the next row, which another wave of the workgroup
    copied in the same window.)"""
    wq, wb, x = _setup(M, N, K, nested, 13 * M + N + K + int(rw) + int(kw))
    keys = ("NF4_GEMV_KW", "NF4_GEMV_RW")
    old = {k: os.environ.get(k) for k in keys}
    os.environ["NF4_GEMV_KW"], os.environ["NF4_GEMV_RW"] = kw, rw
    try:
        xd = x.to(DEV)
        api.nf4_reset_path_counts()
        ys = [api.nf4_matmul_fwd(xd, wq) for _ in range(50)]
        torch.cuda.synchronize()
        c = api.nf4_path_counts()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert c["fwd_small_m"] == 50
    for i, y in enumerate(ys):
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), f"call {i} differs"
    xb = WL.bf16_bits(x)
    assert_close(ys[0], O.matmul_fwd(xb, wb), f"y {M}x{N}x{K} rw={rw} kw={kw}",
                 O.matmul_fwd(abs_bits(xb), abs_bits(wb)), K)
