"""GPU test of nf4_matmul_fwd_noalloc, called through the C ABI: its output
equals nf4_matmul_fwd's (same plan, same kernels, partials in the library's
fixed buffer instead of a caller workspace) bit for bit, on two calls in a row
(the second smaller), and a product needing more partials than the buffer
holds is refused without a launch."""

import ctypes

import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import _lib as L
from nf4_bit_weight_amd import api

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _weight(N, K, seed):
    code = torch.from_numpy(WL.nf4_code_np()).to(DEV)
    ncode = torch.from_numpy(WL.nested_code_np()).to(DEV)
    return api.nf4_quantize(WL.gpu_weight_f32(N, K, seed=seed, device=DEV), code, ncode)


def _noalloc(x, w, y):
    lib = L.lib()
    return lib.nf4_matmul_fwd_noalloc(x.data_ptr(), x.shape[0], w.packed.data_ptr(), w.absmax.data_ptr(),
                                      w.nested_absmax.data_ptr(), w.nested_offset.data_ptr(),
                                      w.code.data_ptr(), w.nested_code.data_ptr(), w.N, w.K,
                                      y.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("first,second", [((512, 4096, 4096), (64, 1024, 4096)),
                                          ((32, 14336, 4096), (8, 4096, 4096))])
def test_noalloc_matches_workspace_call(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        need = api.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, M, N, K)
        assert need <= L.NF4_NOALLOC_SCRATCH_BYTES
        w = _weight(N, K, 95_000 + 10 * M + i)
        x = WL.gpu_normal_bf16(M, K, seed=96_000 + M + i, device=DEV)
        ref = api.nf4_matmul_fwd(x, w)
        y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
        st = _noalloc(x, w, y)
        assert st == L.NF4_OK, L.status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (M, N, K)
    # the first shape's plan splits its contraction: the buffer really carried partials
    assert api.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, *first) > 0


def test_noalloc_refuses_beyond_its_buffer():
    M, N, K = 2048, 5120, 27648
    need = api.nf4_workspace_bytes(L.NF4_OP_MATMUL_FWD, M, N, K)
    assert need > L.NF4_NOALLOC_SCRATCH_BYTES
    w = _weight(N, K, 97_000)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    api.nf4_reset_path_counts()
    assert _noalloc(x, w, y) == L.NF4_ERR_SCRATCH
    torch.cuda.synchronize()
    assert all(v == 0 for v in api.nf4_path_counts().values())
    assert bool((y == 3.0).all())
