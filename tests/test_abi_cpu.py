"""Host-side checks of libnf4.so: it loads, exports every symbol nf4.h
declares, and its host helpers and argument validation behave as documented.
No device work is issued (every call here fails validation or is host-only)."""

import ctypes
import os
import re

import pytest

from nf4_bit_weight_amd import _lib as L
from oracle import nf4_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")

FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from nf4_bit_weight_amd import build as B
        B.build()
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding lacks {n}"


def test_header_macros_match_binding():
    text = open(HEADER).read()
    vals = dict(re.findall(r"#define\s+(NF4_[A-Z0-9_]+)\s+(-?\d+)", text))
    for name in ("NF4_OK", "NF4_ERR_NULL", "NF4_ERR_SHAPE", "NF4_ERR_UNSUPPORTED",
                 "NF4_ERR_ALIGN", "NF4_ERR_WORKSPACE", "NF4_ERR_HIP", "NF4_ERR_DTYPE", "NF4_ERR_SCRATCH",
                 "NF4_DTYPE_F32", "NF4_DTYPE_BF16", "NF4_OP_QUANTIZE", "NF4_OP_MATMUL_FWD",
                 "NF4_OP_MATMUL_BWD_INPUT", "NF4_OP_GROUPED_FWD", "NF4_OP_GROUPED_BWD_INPUT",
                 "NF4_OP_MATMUL_FWD_8BIT", "NF4_OP_MATMUL_BWD_INPUT_8BIT"):
        assert int(vals[name]) == getattr(L, name), name
    assert int(vals["NF4_PATH_COUNT"]) == len(L.PATHS)


def test_storage_helpers_match_oracle(lib):
    for N, K in ((128, 256), (4096, 4096), (27648, 5120), (3, 66), (1, 2)):
        n = N * K
        assert lib.nf4_packed_bytes(N, K) == O.packed_bytes(n)
        assert lib.nf4_absmax_count(N, K) == O.absmax_count(n)
        assert lib.nf4_nested_count(N, K) == O.nested_count(n)
    assert lib.nf4_packed_bytes(-1, 4) == -1


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = L.status_str(code)
        assert s.startswith("NF4_"), s
    assert L.status_str(-99) == "unknown NF4 status"
    assert lib.nf4_version().decode().startswith("nf4-mi355x")


def _fwd(lib, x=FAKE, M=4, packed=FAKE, absmax=FAKE, nabs=None, noff=None, code=FAKE,
         ncode=None, N=8, K=64, y=FAKE, ws=None, wsb=0):
    return lib.nf4_matmul_fwd(x, M, packed, absmax, nabs, noff, code, ncode, N, K, y, ws, wsb, None)


def test_matmul_validation(lib):
    assert _fwd(lib, x=None) == L.NF4_ERR_NULL
    assert _fwd(lib, packed=None) == L.NF4_ERR_NULL
    assert _fwd(lib, code=None) == L.NF4_ERR_NULL
    assert _fwd(lib, nabs=FAKE) == L.NF4_ERR_NULL           # nested without offset/table
    assert _fwd(lib, M=-1) == L.NF4_ERR_SHAPE
    assert _fwd(lib, N=3, K=63) == L.NF4_ERR_SHAPE            # odd element count
    assert _fwd(lib, K=96) == L.NF4_ERR_UNSUPPORTED           # K % 64
    assert _fwd(lib, x=MISALIGNED) == L.NF4_ERR_ALIGN
    assert _fwd(lib, packed=MISALIGNED) == L.NF4_ERR_ALIGN
    assert _fwd(lib, M=0) == L.NF4_OK                         # empty: nothing to do
    assert _fwd(lib, M=0, x=None, y=None) == L.NF4_OK         # empty tensors may be NULL
    assert _fwd(lib, M=0, packed=None) == L.NF4_ERR_NULL      # the weight is still checked
    # a weight with no elements (N = 0) has nothing to point at; the output
    # has no columns, so nothing is launched
    assert _fwd(lib, N=0, packed=None, absmax=None, y=None) == L.NF4_OK
    assert _fwd(lib, N=0, packed=None, absmax=None, code=None) == L.NF4_ERR_NULL
    bw = lib.nf4_matmul_bwd_input(FAKE, 4, FAKE, FAKE, None, None, FAKE, None, 12, 64, FAKE,
                                  None, 0, None)
    assert bw == L.NF4_ERR_UNSUPPORTED                        # N % 8 for the input grad


def test_workspace_is_required_when_planned(lib):
    M, N, K = 512, 1024, 4096
    need = lib.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, M, N, K, 1)
    assert need > 0                                           # small tile count -> split
    assert _fwd(lib, M=M, N=N, K=K) == L.NF4_ERR_WORKSPACE
    assert _fwd(lib, M=M, N=N, K=K, ws=FAKE, wsb=need - 1) == L.NF4_ERR_WORKSPACE
    # the plan is a pure function of the sizes
    assert need == lib.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, M, N, K, 1)
    assert lib.nf4_workspace_bytes(99, 1, 1, 64, 1) == ctypes.c_size_t(-1).value


def test_codec_validation(lib):
    q = lib.nf4_quantize
    assert q(FAKE, 5, 4, 64, FAKE, None, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_DTYPE
    assert q(None, 0, 4, 64, FAKE, None, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_NULL
    assert q(FAKE, 0, 3, 3, FAKE, None, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_SHAPE
    assert q(FAKE, 0, 4, 64, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_NULL
    assert q(FAKE, 0, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == L.NF4_ERR_WORKSPACE
    d = lib.nf4_dequantize
    assert d(FAKE, FAKE, None, None, FAKE, None, 4, 64, 9, FAKE, None) == L.NF4_ERR_DTYPE
    assert d(FAKE, FAKE, None, None, FAKE, None, 4, 64, 1, None, None) == L.NF4_ERR_NULL


def test_grouped_validation(lib):
    g = lib.nf4_grouped_matmul_fwd
    assert g(FAKE, FAKE, 0, 8, FAKE, FAKE, None, None, FAKE, None, 8, 64, FAKE, None, 0, None) == L.NF4_ERR_SHAPE
    assert g(FAKE, None, 2, 8, FAKE, FAKE, None, None, FAKE, None, 8, 64, FAKE, None, 0, None) == L.NF4_ERR_NULL
    assert g(FAKE, FAKE, 2, 8, FAKE, FAKE, None, None, FAKE, None, 8, 96, FAKE, None, 0, None) == L.NF4_ERR_UNSUPPORTED
    assert g(None, FAKE, 2, 0, FAKE, FAKE, None, None, FAKE, None, 8, 64, None, None, 0, None) == L.NF4_OK
    assert g(None, FAKE, 2, 4, FAKE, FAKE, None, None, FAKE, None, 8, 64, FAKE, None, 0, None) == L.NF4_ERR_NULL


def test_path_counters_host_side(lib):
    lib.nf4_reset_path_counts()
    for p in range(len(L.PATHS)):
        assert lib.nf4_path_count(p) == 0
    assert lib.nf4_path_count(len(L.PATHS)) == -1
    _fwd(lib, x=None)                                         # a rejected call counts nothing
    assert lib.nf4_path_count(2) == 0


def test_library_has_no_undefined_internal_symbols():
    """Every kernel the library launches is defined in it (a kernel whose
    host-side launch stub is missing would leave an undefined symbol that
    only fails when the library is loaded on the GPU host)."""
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    from nf4_bit_weight_amd import _lib

    out = subprocess.run([nm, "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    bad = [ln for ln in out.splitlines() if "nf4" in ln]
    assert not bad, bad


def test_no_memset_in_library_sources():
    """The library zeroes with its own kernel, never hipMemset*: a caller may
    capture any entry point into a HIP graph, and a captured memset node is
    avoided on this target."""
    csrc = os.path.join(ROOT, "nf4_bit_weight_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, name)).read()
        code = re.sub(r"//[^\n]*", "", re.sub(r"/\*.*?\*/", "", text, flags=re.S))
        assert not re.search(r"\bhipMemset\w*\s*\(", code), f"{name} calls hipMemset"


def test_noalloc_validation(lib):
    """The no-allocation forward validates like nf4_matmul_fwd and refuses a
    plan whose partials exceed its fixed buffer before touching the device."""
    def f(x=FAKE, M=4, packed=FAKE, N=8, K=64, y=FAKE):
        return lib.nf4_matmul_fwd_noalloc(x, M, packed, FAKE, None, None, FAKE, None, N, K, y, None)
    assert f(x=None) == L.NF4_ERR_NULL
    assert f(K=96) == L.NF4_ERR_UNSUPPORTED
    assert f(M=0) == L.NF4_OK
    M, N, K = 2048, 5120, 27648
    assert lib.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, M, N, K, 1) > L.NF4_NOALLOC_SCRATCH_BYTES
    assert f(M=M, N=N, K=K) == L.NF4_ERR_SCRATCH
    text = open(HEADER).read()
    assert f"#define NF4_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert L.NF4_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_8bit_validation(lib):
    """The 8-bit entry points validate like the 4-bit ones; an odd element
    count is allowed (one byte per weight) and the 8-bit workspace comes from
    its own op codes."""
    def f(x=FAKE, M=4, packed=FAKE, N=8, K=64, y=FAKE, ws=None, wsb=0):
        return lib.nf4_matmul_fwd_8bit(x, M, packed, FAKE, None, None, FAKE, None, N, K, y, ws, wsb, None)
    assert f(x=None) == L.NF4_ERR_NULL
    assert f(packed=None) == L.NF4_ERR_NULL
    assert f(K=96) == L.NF4_ERR_UNSUPPORTED
    assert f(M=0) == L.NF4_OK
    q = lib.nf4_quantize_8bit
    assert q(None, 0, 3, 5, FAKE, None, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_NULL
    assert q(FAKE, 9, 4, 64, FAKE, None, FAKE, FAKE, None, None, None, 0, None) == L.NF4_ERR_DTYPE
    M, N, K = 8, 1024, 4096
    need = lib.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD_8BIT, M, N, K, 1)
    assert need > 0                                          # few tiles: contraction split
    assert f(M=M, N=N, K=K) == L.NF4_ERR_WORKSPACE
    assert lib.nf4_workspace_bytes(L.NF4_OP_MATMUL_BWD_INPUT_8BIT, 0, N, K, 1) == 0
    d = lib.nf4_dequantize_8bit
    assert d(FAKE, FAKE, None, None, FAKE, None, 4, 64, 7, FAKE, None) == L.NF4_ERR_DTYPE
