"""Host-side checks of the layer-buffer and slot logic (no GPU).

The layer buffer (used by the aliasing harness and the layer streamer) must
reproduce every field bit for bit through its views and keep every field
aligned; the harness's slot ring must hand out slots round-robin,
overwriting the one handed out ``n_slots`` acquires earlier.
"""

import numpy as np
import torch

import aliasing_harness as AH
from nf4_bit_weight_amd import streaming
from nf4_bit_weight_amd.api import NF4Weight


def _fake_weight(N, K, seed, nested=True):
    g = np.random.default_rng(seed)
    nb = N * K // 64
    packed = torch.from_numpy(g.integers(0, 256, N * K // 2, dtype=np.uint8))
    code = torch.linspace(-1, 1, 16)
    if nested:
        ng = (nb + 255) // 256
        return NF4Weight(packed, torch.from_numpy(g.integers(0, 256, nb, dtype=np.uint8)),
                         torch.from_numpy(g.random(ng, dtype=np.float32)),
                         torch.tensor([0.25], dtype=torch.float32), code, torch.linspace(-1, 1, 256), N, K)
    return NF4Weight(packed, torch.from_numpy(g.random(nb, dtype=np.float32)), None, None, code, None, N, K)


def test_packed_layer_roundtrip_and_alignment():
    for nested in (True, False):
        ws = [_fake_weight(N, K, i, nested) for i, (N, K) in enumerate([(128, 192), (64, 4160), (200, 64)])]
        lay = AH.PackedLayer(["a", "b", "c"], ws)
        for buf in (lay.store, lay.store.clone()):
            views = lay.views(buf)
            for name, w in zip("abc", ws):
                v = views[name]
                assert (v.N, v.K) == (w.N, w.K)
                for got, want in zip(v.tensors()[:4], w.tensors()[:4]):
                    if want is None:
                        assert got is None
                        continue
                    assert got.dtype == want.dtype and got.shape == want.shape
                    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
                    assert (got.data_ptr() - buf.data_ptr()) % streaming.ALIGN == 0
        assert lay.nbytes >= sum(w.nbytes() for w in ws)


def test_views_alias_the_buffer():
    ws = [_fake_weight(64, 128, 7)]
    lay = AH.PackedLayer(["a"], ws)
    buf = lay.store.clone()
    v = lay.views(buf)["a"]
    buf.zero_()
    assert int(v.packed.sum()) == 0 and int(v.absmax.sum()) == 0


def test_dense_layer_views():
    d = [torch.randn(8, 16).to(torch.bfloat16), torch.randn(3, 5).to(torch.bfloat16)]
    lay = AH.DenseLayer(["x", "y"], d)
    v = lay.views(lay.store)
    assert torch.equal(v["x"], d[0]) and torch.equal(v["y"], d[1])


def test_slot_ring_round_robin():
    src = [torch.full((4,), float(i)) for i in range(5)]
    ring = AH.SlotRing(2, src[0])
    got = [ring.acquire(s) for s in src]
    assert got[0] is got[2] is got[4] and got[1] is got[3]
    # what a holder of the first slot sees after the later acquires
    assert torch.equal(got[0], src[4]) and torch.equal(got[1], src[3])


def test_layer_buffer_rejects_small_or_wrong_buffers():
    import pytest
    lay = streaming.LayerBuffer(["a"], [_fake_weight(64, 128, 8)])
    with pytest.raises(ValueError):
        lay.views(lay.store[:-1])
    with pytest.raises(ValueError):
        lay.views(torch.zeros(lay.nbytes, dtype=torch.int8))
