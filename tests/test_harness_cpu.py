"""Host-side checks of the layer-buffer and slot logic (no GPU).

The layer buffer (used by the aliasing harness and the layer streamer) must
reproduce every field bit for bit through its views and keep every field
aligned; the harness's slot schedule must send fill f to slot f mod n, so a
reused slot holds the bytes of the latest fill that landed in it.
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
        lay = streaming.LayerBuffer(["a", "b", "c"], ws)
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
    lay = streaming.LayerBuffer(["a"], ws)
    buf = lay.store.clone()
    v = lay.views(buf)["a"]
    buf.zero_()
    assert int(v.packed.sum()) == 0 and int(v.absmax.sum()) == 0


def test_dense_block_store_views():
    d = [torch.randn(8, 16).to(torch.bfloat16), torch.randn(3, 5).to(torch.bfloat16)]
    lay = AH.DenseBlockStore(["x", "y"], d)
    v = lay.views(lay.store)
    assert torch.equal(v["x"], d[0]) and torch.equal(v["y"], d[1])
    assert all((s * 2) % streaming.ALIGN == 0 for s in lay.starts)


def test_slot_schedule_and_weight_source():
    sched = AH.SlotSchedule(3)
    assert [sched.next_slot() for _ in range(7)] == [0, 1, 2, 0, 1, 2, 0]
    d = [[torch.full((4, 4), float(i)).to(torch.bfloat16)] for i in range(5)]
    stores = [AH.DenseBlockStore(["w"], b) for b in d]
    src = AH.WeightSource(stores, reuse=True, n_slots=2)
    got = [src.weights(i)["w"] for i in range(5)]
    # fills 0, 2, 4 share slot 0 and fills 1, 3 slot 1: an early holder sees the latest fill
    assert got[0].data_ptr() == got[2].data_ptr() == got[4].data_ptr()
    assert got[1].data_ptr() == got[3].data_ptr() != got[0].data_ptr()
    assert torch.equal(got[0], d[4][0]) and torch.equal(got[1], d[3][0])
    own = AH.WeightSource(stores, reuse=False, n_slots=2)
    assert [float(own.weights(i)["w"][0, 0]) for i in range(5)] == [0.0, 1.0, 2.0, 3.0, 4.0]
    assert own.weights(2)["w"].data_ptr() == stores[2].store.data_ptr()


def test_layer_buffer_rejects_small_or_wrong_buffers():
    import pytest
    lay = streaming.LayerBuffer(["a"], [_fake_weight(64, 128, 8)])
    with pytest.raises(ValueError):
        lay.views(lay.store[:-1])
    with pytest.raises(ValueError):
        lay.views(torch.zeros(lay.nbytes, dtype=torch.int8))
