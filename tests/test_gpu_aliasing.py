"""GPU tests of the checkpoint-visible wrapper under weight aliasing.

bitsandbytes issue #2034 ("Minimal reproducer", "What it prints", "Why
save_for_backward fixes it") and Soup issue #842 ("Acceptance criteria"):

* with 2 reused slots for 8 Qwen-32B-shaped layers (~240 MiB of nested NF4
  each, above the ~165 MiB of Soup #842 "The constraint: #331"), the fused
  wrapper's gradients are bit-identical to those with a private buffer per
  layer, and so are the dense bf16 control's;
* the negative control (same kernels, weight fields held on ctx) gets every
  gradient wrong except those of the last ``slots`` layers, while its forward
  loss stays bit-exact -- the pattern #2034 prints;
* without checkpointing, overwriting a saved weight buffer in place between
  forward and backward raises autograd's version-counter error for the
  wrapper, and silently changes the negative control's gradient;
* a saved_tensors_hooks audit (Experts PR, "Commit 2") finds nothing
  weight-shaped saved by the plain or the grouped wrapper, while a
  dequantise + F.linear control does save the dense weight.
"""

import pytest
import torch
import torch.nn.functional as F

import aliasing_harness as AH
import workloads as WL
from nf4_bit_weight_amd import api
from nf4_bit_weight_amd.autograd import nf4_grouped_linear, nf4_linear

pytestmark = pytest.mark.gpu

LAYERS = 8


@pytest.fixture(scope="module")
def model():
    m = AH.make_workload(layers=LAYERS, tokens=256)
    yield m
    del m
    torch.cuda.empty_cache()


def test_layer_size_above_threshold(model):
    assert model.packed[0].nbytes > 165 * 2 ** 20


@pytest.mark.parametrize("arm", ["fused", "dense"])
def test_reused_equals_private(model, arm):
    p = AH.train_step(model, arm, reuse=False)
    r = AH.train_step(model, arm, reuse=True)
    assert torch.equal(p.loss, r.loss), f"{arm}: forward loss differs"
    for i, (a, b) in enumerate(zip(r.grads, p.grads)):
        assert torch.equal(a, b), f"{arm}: gradient {i} differs with reused slots"


@pytest.mark.parametrize("slots", [2, 3])
def test_negative_control_pattern(model, slots):
    p = AH.train_step(model, "ctx_held", reuse=False, slots=slots)
    r = AH.train_step(model, "ctx_held", reuse=True, slots=slots)
    assert torch.equal(p.loss, r.loss), "forward must stay bit-exact"
    gp = p.grads
    d = AH.grad_gaps(r, p)
    for i in range(LAYERS - slots):
        # wrong by far more than rounding: another layer's weights were used
        rel = d[i] / float(gp[i].float().abs().max().item())
        assert rel > 0.05, f"layer {i}: negative control not detected ({d[i]:.3e})"
    for i in range(LAYERS - slots, LAYERS):
        assert d[i] == 0.0, f"layer {i}: slot not yet recycled, must be exact"
    assert d[LAYERS] > 0.0, "input gradient passes through recycled layers"
    # with private buffers the two wrappers run the same kernels on the same bytes
    gf = AH.train_step(model, "fused", reuse=False, slots=slots).grads
    for i, (a, b) in enumerate(zip(gf, gp)):
        assert torch.equal(a, b), f"private arms differ at {i}"


def test_without_early_stop(model):
    # every recompute replays the slot copy: the wrapper stays exact, the
    # negative control now reads the next layer's bytes everywhere but last
    p = AH.train_step(model, "fused", reuse=False, early_stop=False)
    r = AH.train_step(model, "fused", reuse=True, early_stop=False)
    assert torch.equal(p.loss, r.loss)
    assert all(torch.equal(a, b) for a, b in zip(r.grads, p.grads))
    cp = AH.train_step(model, "ctx_held", reuse=False, early_stop=False)
    cr = AH.train_step(model, "ctx_held", reuse=True, early_stop=False)
    d = AH.grad_gaps(cr, cp)
    assert all(v > 0 for v in d[:LAYERS - 1]) and d[LAYERS - 1] == 0.0, d


def test_version_counter_catches_overwrite(model):
    l0, l1 = model.packed[0], model.packed[1]
    slot = l0.store.clone()
    x = model.x.clone().requires_grad_(True)
    y = nf4_linear(x, l0.views(slot)["q"])
    slot.copy_(l1.store)                                 # in-place overwrite of the saved bytes
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        torch.sum(y.float() ** 2).backward()

    # the negative control computes with whatever the slot now holds
    slot.copy_(l0.store)
    xr = model.x.clone().requires_grad_(True)
    yr = nf4_linear(xr, l0.views(l0.store)["q"])
    torch.sum(yr.float() ** 2).backward()
    xc = model.x.clone().requires_grad_(True)
    yc = AH.CtxHeldNF4MatMul.apply(xc, [l0.views(slot)["q"]])
    slot.copy_(l1.store)
    torch.sum(yc.float() ** 2).backward()
    torch.cuda.synchronize()
    assert torch.equal(yc, yr), "forward identical"
    assert not torch.equal(xc.grad, xr.grad), "negative control must be silently wrong"


def _audit(fn):
    saved = []

    def pack(t):
        saved.append(t)
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        out = fn()
    return out, saved


def test_saved_tensors_audit_linear(model):
    lay = model.packed[0]
    w = lay.views(lay.store)["gate"]
    N, K = w.N, w.K
    x = model.x.clone().requires_grad_(True)
    _, saved = _audit(lambda: nf4_linear(x, w))
    shapes = {tuple(t.shape) for t in saved}
    assert (N, K) not in shapes and (K, N) not in shapes
    assert not any(t.is_floating_point() and t.numel() >= N * K // 64 for t in saved)
    code_bytes = (16 + 256) * 4
    assert sum(t.numel() * t.element_size() for t in saved) == w.nbytes() + code_bytes
    # control: dequantise + F.linear saves the dense weight
    _, saved_c = _audit(lambda: F.linear(x, api.nf4_dequantize(w)))
    shapes_c = {tuple(t.shape) for t in saved_c}
    assert (N, K) in shapes_c or (K, N) in shapes_c


def test_saved_tensors_audit_grouped():
    E, H, I = WL.OLMOE_E, WL.OLMOE_HIDDEN, WL.OLMOE_INTER
    dev = torch.device("cuda:0")
    code = torch.from_numpy(WL.nf4_code_np()).to(dev)
    ncode = torch.from_numpy(WL.nested_code_np()).to(dev)
    w = api.nf4_quantize(WL.gpu_weight_f32(E * I, H, seed=83_000, device=dev), code, ncode).per_expert(E)
    _, _, offsets = WL.olmoe_routing()
    off = torch.from_numpy(offsets).to(dev)
    T = int(offsets[-1])
    x = WL.gpu_normal_bf16(T, H, seed=83_001, device=dev).requires_grad_(True)
    y, saved = _audit(lambda: nf4_grouped_linear(x, off, w, E))
    weight_shapes = {(I, H), (H, I), (E, I, H), (E, H, I), (E * I, H), (H, E * I)}
    assert not ({tuple(t.shape) for t in saved} & weight_shapes)
    assert not any(t.is_floating_point() and t.numel() >= I * H // 64 for t in saved)
    y.float().sum().backward()
    assert x.grad is not None and torch.isfinite(x.grad.float()).all()
    # control: per-expert dequantise + F.linear saves weight-shaped tensors
    wd = api.nf4_dequantize(api.NF4Weight(*w.tensors(), E * I, H)).view(E, I, H)

    def dense():
        outs = [F.linear(x[offsets[e]:offsets[e + 1]], wd[e]) for e in range(E)]
        return torch.cat(outs)

    _, saved_c = _audit(dense)
    assert {tuple(t.shape) for t in saved_c} & weight_shapes
