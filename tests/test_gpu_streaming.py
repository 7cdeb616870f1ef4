"""Layer streaming through a ring of device slots (Soup issue #842,
"Acceptance criteria": streamed vs resident NF4, both arms on the new kernel,
forward and backward stated separately).

Llama-3.1-8B-shaped layers live in page-locked host memory and are copied
into 2 or 3 device slots on every visit (forward in layer order, then the
input gradients in reverse).  Every forward and every input gradient must be
bit-identical to the same step run on device-resident weights, and repeat
bit for bit; the streamer must have copied each layer exactly twice.
"""

import pytest
import torch

import workloads as WL
from nf4_bit_weight_amd import api
from nf4_bit_weight_amd.streaming import LayerBuffer, SlotStreamer

pytestmark = pytest.mark.gpu

L = 4
M = 256
PROJS = WL.LLAMA_8B
NAMES = [p.name for p in PROJS]


@pytest.fixture(scope="module")
def stack():
    dev = torch.device("cuda:0")
    code = torch.from_numpy(WL.nf4_code_np()).to(dev)
    ncode = torch.from_numpy(WL.nested_code_np()).to(dev)
    resident, host = [], []
    for l in range(L):
        ws = []
        for i, p in enumerate(PROJS):
            w = WL.gpu_weight_f32(p.N, p.K, seed=84_000 + 16 * l + i, device=dev)
            ws.append(api.nf4_quantize(w, code, ncode))
            del w
        resident.append(LayerBuffer(NAMES, ws))
        host.append(LayerBuffer(NAMES, ws, pin_memory=True))
        del ws
    xs = [[WL.gpu_normal_bf16(M, p.K, seed=85_000 + 16 * l + i, device=dev) for i, p in enumerate(PROJS)]
          for l in range(L)]
    gys = [[WL.gpu_normal_bf16(M, p.N, seed=86_000 + 16 * l + i, device=dev) for i, p in enumerate(PROJS)]
           for l in range(L)]
    torch.cuda.synchronize()
    return resident, host, xs, gys


VISITS = list(range(L)) + list(reversed(range(L)))


def _step(xs, gys, out):
    def fn(v, layer, w):
        if v < L:
            out[("fwd", layer)] = [api.nf4_matmul_fwd(xs[layer][i], w[n]) for i, n in enumerate(NAMES)]
        else:
            out[("bwd", layer)] = [api.nf4_matmul_bwd_input(gys[layer][i], w[n]) for i, n in enumerate(NAMES)]
    return fn


def _resident_step(resident, xs, gys):
    out = {}
    fn = _step(xs, gys, out)
    for v, layer in enumerate(VISITS):
        fn(v, layer, resident[layer].views(resident[layer].store))
    torch.cuda.synchronize()
    return out


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        for i, (u, w) in enumerate(zip(a[k], b[k])):
            assert torch.equal(u.view(torch.int16), w.view(torch.int16)), f"{k} projection {NAMES[i]}"


@pytest.mark.parametrize("slots", [2, 3])
def test_streamed_equals_resident(stack, slots):
    resident, host, xs, gys = stack
    want = _resident_step(resident, xs, gys)
    st = SlotStreamer(host, slots, torch.device("cuda:0"))
    for rep in range(2):
        got = {}
        st.run(VISITS, _step(xs, gys, got))
        torch.cuda.synchronize()
        _same(got, want)
    assert st.bytes_copied == 2 * 2 * sum(h.nbytes for h in host)
    assert st.device_bytes == slots * max(h.nbytes for h in host)


def test_host_buffers_are_pinned_and_match(stack):
    resident, host, _, _ = stack
    for r, h in zip(resident, host):
        assert h.store.is_pinned() and not h.store.is_cuda
        assert torch.equal(h.store, r.store.cpu())
