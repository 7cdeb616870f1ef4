"""Weight-aliasing harness for the checkpoint-visible NF4 wrapper.

bitsandbytes issue #2034 ("Minimal reproducer", "What it prints", "Root
cause") and Soup issue #842 ("Acceptance criteria", aliasing control): a
streaming caller copies each layer's packed weight into a small ring of
recycled device buffers inside a non-reentrant ``torch.utils.checkpoint``
region.  A wrapper that routes every weight field through
``save_for_backward`` gets the recompute's freshly copied bytes in backward;
a wrapper that keeps them on ctx as attributes reads whatever a later copy
left in the slot, so its input gradients come out wrong while the forward
stays bit-exact.

Arms (each run twice, with recycled slots and with a private buffer per
layer, then compared gradient by gradient):

* ``fused``: ``nf4_linear`` (the fused kernels, every field saved through
  ``save_for_backward``);
* ``dense``: the same layers as dense bf16 ``W_hat`` through ``F.linear`` --
  the control showing that the harness itself is sound;
* ``ctx_held``: the negative control, the same fused kernels behind a
  Function that keeps the weight fields on ctx.  Under recycling only the
  last ``slots`` layers may come out right.

A layer is the seven projections of a Qwen-32B-shaped block in nested NF4
(about 240 MiB of packed fields), above the ~165 MiB per layer at which
Soup #842 ("The constraint: #331") saw the wrong gradients.  Each projection
consumes either the layer input h or another projection's output, and the
layer's output is a fixed linear combination of them, so nothing after the
slot copy is saved by autograd except what the projection wrappers save --
the non-reentrant recompute therefore replays the slot copy exactly when the
wrapper saved its weight fields (Soup #842 and #1999 describe the recompute
stopping early once the last saved tensor is rebuilt).

Run as a script on a GPU to print the per-layer table:
    python tests/aliasing_harness.py
"""

from __future__ import annotations

import os
import sys
from dataclasses import dataclass

if __name__ == "__main__":                       # run as a script: the repository root holds the packages
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch
import torch.nn.functional as F
from torch.utils.checkpoint import checkpoint

import workloads as WL
from nf4_bit_weight_amd import api
from nf4_bit_weight_amd.autograd import nf4_linear
from nf4_bit_weight_amd.streaming import LayerBuffer

ALIGN = 256          # alignment of every dense block inside a layer buffer


def _round_up(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


# One layer's NF4 fields in a single byte buffer, so a slot copy moves the
# whole layer with one copy_; views(buf) rebuilds the projections on a slot.
PackedLayer = LayerBuffer


class DenseLayer:
    """The same layer as dense bf16 W_hat [N, K] blocks in one buffer."""

    def __init__(self, names, dense):
        self.names = list(names)
        self.shapes = [tuple(d.shape) for d in dense]
        self.offsets = []
        off = 0
        for d in dense:
            self.offsets.append(off)
            off += _round_up(d.numel())
        self.store = torch.empty(off, dtype=torch.bfloat16, device=dense[0].device)
        for d, o in zip(dense, self.offsets):
            self.store[o:o + d.numel()].copy_(d.reshape(-1))

    def views(self, buf: torch.Tensor) -> dict:
        return {n: buf[o:o + s[0] * s[1]].view(s) for n, o, s in zip(self.names, self.offsets, self.shapes)}


class SlotRing:
    """Round-robin recycled device buffers: every ``acquire`` copies the
    source into the next slot and hands that slot out, so a slot given out in
    the original forward is overwritten later in the same step."""

    def __init__(self, n_slots: int, like: torch.Tensor):
        self.slots = [torch.empty_like(like) for _ in range(n_slots)]
        self.cursor = 0

    def acquire(self, src: torch.Tensor) -> torch.Tensor:
        slot = self.slots[self.cursor % len(self.slots)]
        self.cursor += 1
        slot.copy_(src)
        return slot


class CtxHeldNF4MatMul(torch.autograd.Function):
    """Negative control: the same fused kernels, with the weight fields kept
    on ctx as plain attributes instead of ``save_for_backward`` (the pattern
    bitsandbytes #2034 "Root cause" describes).  Checkpointing never sees
    them, so a recycled slot is read back as whatever it holds at backward
    time.  Never use this outside the harness."""

    @staticmethod
    def forward(ctx, x, w_holder):
        w = w_holder[0]
        ctx.w = w
        return api.nf4_matmul_fwd(x.contiguous(), w)

    @staticmethod
    def backward(ctx, grad_y):
        return api.nf4_matmul_bwd_input(grad_y.contiguous(), ctx.w), None


def _linear(arm: str):
    if arm == "fused":
        return nf4_linear
    if arm == "ctx_held":
        return lambda x, w: CtxHeldNF4MatMul.apply(x, [w])
    if arm == "dense":
        return F.linear
    raise ValueError(arm)


def layer_forward(x, h, weights: dict, lin):
    """One block after its trainable scale (h = x * scale, computed upstream
    of the weight copy, so the scale's gradient is computed from W in the
    backward): the seven projections combined linearly.  k and v (N = 1024)
    are tiled back to the model width as grouped-query heads are."""
    q = lin(h, weights["q"])
    k = lin(h, weights["k"])
    v = lin(h, weights["v"])
    a = lin(q, weights["o"])
    g = lin(h, weights["gate"]) + lin(h, weights["up"])
    d = lin(g, weights["down"])
    rep = q.shape[1] // k.shape[1]
    return x + 0.05 * (a + d + (k + v).repeat(1, rep))


@dataclass
class HarnessModel:
    nf4_layers: list
    dense_layers: list
    x: torch.Tensor
    scales_init: list


def build(layers: int = 8, tokens: int = 256, projs=WL.QWEN_32B, seed: int = 0,
          dense: bool = True, device="cuda") -> HarnessModel:
    """Seeded synthetic layers: weights 0.02 N(0,1) quantised to nested NF4
    on the device; the dense control gets the dequantised W_hat of the same
    weights, so both arms multiply by identical values."""
    code = torch.from_numpy(WL.nf4_code_np()).to(device)
    ncode = torch.from_numpy(WL.nested_code_np()).to(device)
    names = [p.name for p in projs]
    nf4_layers, dense_layers = [], []
    for l in range(layers):
        ws, ds = [], []
        for i, p in enumerate(projs):
            w = WL.gpu_weight_f32(p.N, p.K, seed=80_000 + 100 * seed + 16 * l + i, device=device)
            q = api.nf4_quantize(w, code, ncode)
            del w
            ws.append(q)
            if dense:
                ds.append(api.nf4_dequantize(q))
        nf4_layers.append(PackedLayer(names, ws))
        del ws
        if dense:
            dense_layers.append(DenseLayer(names, ds))
            del ds
    width = projs[0].K
    x = WL.gpu_normal_bf16(tokens, width, seed=81_000 + seed, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(82_000 + seed)
    scales = [(1.0 + 0.01 * torch.randn(width, generator=gen, device=device)).to(torch.bfloat16)
              for _ in range(layers)]
    torch.cuda.synchronize()
    return HarnessModel(nf4_layers, dense_layers, x, scales)


def run(model: HarnessModel, arm: str, recycle: bool, slots: int = 2, use_checkpoint: bool = True,
        early_stop: bool = True):
    """One forward + backward through every layer.  Returns (loss, grads)
    with grads = [grad of each layer's scale] + [grad of the input].

    With early stop (torch's default), a layer's recompute ends once the
    tensors its forward saved are rebuilt: for the negative control that is
    before the slot copy, so the slots keep their last forward contents and
    the last ``slots`` layers come out right.  Without it every recompute
    replays the copy before the ctx-held backward reads the slot, and only
    the last layer does."""
    layers = model.dense_layers if arm == "dense" else model.nf4_layers
    ring = SlotRing(slots, layers[0].store) if recycle else None
    lin = _linear(arm)
    params = [s.clone().requires_grad_(True) for s in model.scales_init]
    x0 = model.x.clone().requires_grad_(True)

    def body(idx):
        def fn(x, scale):
            h = x * scale                      # trainable, before the weight copy
            # the copy sits inside the checkpointed region: a recompute that
            # runs past this point copies the layer into the next slot again
            buf = ring.acquire(layers[idx].store) if recycle else layers[idx].store
            return layer_forward(x, h, layers[idx].views(buf), lin)
        return fn

    x = x0
    for i in range(len(layers)):
        if use_checkpoint:
            x = checkpoint(body(i), x, params[i], use_reentrant=False, early_stop=early_stop)
        else:
            x = body(i)(x, params[i])
    loss = x.float().pow(2).mean()
    loss.backward()
    torch.cuda.synchronize()
    return loss.detach().clone(), [p.grad.detach().clone() for p in params] + [x0.grad.detach().clone()]


def max_abs_diffs(a, b):
    return [float((u.float() - v.float()).abs().max().item()) for u, v in zip(a, b)]


def table(model: HarnessModel, slots: int = 2):
    """{arm: (loss recycled == loss private, per-layer max |grad diff|)}."""
    out = {}
    for arm in ("fused", "dense", "ctx_held"):
        if arm == "dense" and not model.dense_layers:
            continue
        lp, gp = run(model, arm, recycle=False, slots=slots)
        lr, gr = run(model, arm, recycle=True, slots=slots)
        out[arm] = (bool(torch.equal(lp, lr)), max_abs_diffs(gr, gp))
    return out


def main(argv):
    model = build()
    mib = model.nf4_layers[0].nbytes / 2 ** 20
    res = table(model)
    print(f"layer buffer: {mib:.1f} MiB nested NF4, 2 slots for {len(model.nf4_layers)} layers")
    print(f"{'layer':>5}  " + "  ".join(f"{a + ' recycled vs private':>28}" for a in res))
    n = len(model.nf4_layers)
    for i in range(n + 1):
        name = str(i) if i < n else "x"
        print(f"{name:>5}  " + "  ".join(f"{d[i]:>22.6e} {'MISMATCH' if d[i] else '  ok    '}"
                                         for (_, d) in res.values()))
    print("forward loss bit-equal: " + ", ".join(f"{a}={e}" for a, (e, _) in res.items()))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
