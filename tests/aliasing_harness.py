"""Weight-aliasing harness for the checkpoint-visible NF4 wrapper.

What it checks comes from bitsandbytes issue #2034 ("Minimal reproducer",
"What it prints", "Root cause") and Soup issue #842 ("Acceptance criteria",
the aliasing control).  A streaming caller fills a small set of reused
device slots with each layer's packed weight, and the fill happens inside a
non-reentrant ``torch.utils.checkpoint`` region.  The recompute therefore
fills a slot again, and that slot is not necessarily the one the original
forward used.  A wrapper whose weight fields travel through
``save_for_backward`` gets the recompute's bytes in its backward.  A wrapper
that keeps them as ctx attributes reads whatever the slot holds by then.
Its input gradients are wrong, while its forward is bit-exact.

The harness is this project's own: a ``SlotSchedule`` decides which slot
each fill goes to, a ``WeightSource`` owns the slots (or hands every layer its
own buffer), and a ``Block`` runs one layer from the weights the source
materialises.  One training step multiplies every layer's input by a
trainable gain vector, runs the blocks under non-reentrant checkpointing and
back-propagates a fixed random projection of the output.  The gains'
gradients are computed from the weights in the backward, so they expose
which bytes the backward read.

Arms, each run with reused slots and with a private buffer per layer:

* ``fused``: ``nf4_linear`` (every field through ``save_for_backward``);
* ``dense``: the same layers as dense bf16 ``W_hat`` through ``F.linear``
  (the control that shows the harness is sound);
* ``ctx_held``: the negative control, the same fused kernels behind a
  Function that keeps the weight fields on ctx (the #2034 pattern).

A layer is a Qwen-32B-shaped block of seven projections in nested NF4 (about
240 MiB of packed fields), above the ~165 MiB per layer at which Soup #842
("The constraint: #331") saw wrong gradients.

Run as a script on a GPU for the per-layer summary:
    python tests/aliasing_harness.py
"""

from __future__ import annotations

import os
import sys
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

if __name__ == "__main__":                       # run as a script: the repository root holds the packages
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch
import torch.nn.functional as F
from torch.utils.checkpoint import checkpoint

import workloads as WL
from nf4_bit_weight_amd import api
from nf4_bit_weight_amd.autograd import nf4_linear
from nf4_bit_weight_amd.streaming import ALIGN, LayerBuffer

ARMS = ("fused", "dense", "ctx_held")


class DenseBlockStore:
    """A layer's dense bf16 W_hat blocks [N, K] in one flat buffer, each block
    starting on an ALIGN-byte boundary (the dense twin of ``LayerBuffer``)."""

    def __init__(self, names, blocks: List[torch.Tensor]):
        self.names = list(names)
        self.shapes = [tuple(b.shape) for b in blocks]
        step = ALIGN // 2                               # bf16 elements per ALIGN bytes
        starts, pos = [], 0
        for b in blocks:
            starts.append(pos)
            pos += -(-b.numel() // step) * step
        self.starts = starts
        self.store = torch.zeros(pos, dtype=torch.bfloat16, device=blocks[0].device)
        for b, s in zip(blocks, starts):
            self.store.narrow(0, s, b.numel()).copy_(b.flatten())

    @property
    def nbytes(self) -> int:
        return self.store.numel() * 2

    def views(self, buf: torch.Tensor) -> Dict[str, torch.Tensor]:
        return {n: buf.narrow(0, s, r * c).view(r, c)
                for n, s, (r, c) in zip(self.names, self.starts, self.shapes)}


class SlotSchedule:
    """Which of ``n`` slots the next fill goes to: fill number f uses slot
    f mod n.  The count runs on across the forward and the recompute, as a
    streaming caller's does, so the recompute of a layer generally lands in
    a different slot than its forward did."""

    def __init__(self, n: int):
        if n < 1:
            raise ValueError("at least one slot")
        self.n = n
        self.fills = 0

    def next_slot(self) -> int:
        k = self.fills % self.n
        self.fills += 1
        return k


class WeightSource:
    """Materialises a layer's weights for one visit.  Reused mode: the layer's
    bytes are copied into the slot the schedule names and views of that slot
    are returned.  Private mode: views of the layer's own buffer, nothing is
    ever overwritten."""

    def __init__(self, stores, reuse: bool, n_slots: int):
        self.stores = list(stores)
        self.reuse = reuse
        self.schedule = SlotSchedule(n_slots)
        if reuse:
            size = max(s.store.numel() for s in self.stores)
            proto = self.stores[0].store
            self.slots = [torch.empty(size, dtype=proto.dtype, device=proto.device)
                          for _ in range(n_slots)]
        else:
            self.slots = []

    def weights(self, layer: int) -> dict:
        src = self.stores[layer]
        if not self.reuse:
            return src.views(src.store)
        dst = self.slots[self.schedule.next_slot()].narrow(0, 0, src.store.numel())
        dst.copy_(src.store)
        return src.views(dst)


class CtxHeldNF4MatMul(torch.autograd.Function):
    """Negative control: the fused kernels with the weight fields kept on ctx
    as an attribute instead of through ``save_for_backward`` (the pattern of
    bitsandbytes #2034 "Root cause").  Checkpointing never re-materialises
    them, so a reused slot is read back with whatever it holds at backward
    time.  Only for this harness."""

    @staticmethod
    def forward(ctx, x, holder):
        ctx.weight = holder[0]
        return api.nf4_matmul_fwd(x.contiguous(), holder[0])

    @staticmethod
    def backward(ctx, grad_y):
        return api.nf4_matmul_bwd_input(grad_y.contiguous(), ctx.weight), None


def projection(arm: str) -> Callable:
    return {
        "fused": nf4_linear,
        "dense": F.linear,
        "ctx_held": lambda x, w: CtxHeldNF4MatMul.apply(x, [w]),
    }[arm]


def mix(x, u, w: dict, lin) -> torch.Tensor:
    """One block on the gained input u: attention-like q -> o, grouped k/v
    heads tiled to the width, a gate/up sum -> down, added to the residual x
    with a small weight.  Every projection reads u or another projection's
    output, so the block saves nothing weight-dependent outside the wrapper."""
    q = lin(u, w["q"])
    kv = lin(u, w["k"]) + lin(u, w["v"])
    attn = lin(q, w["o"])
    ffn = lin(lin(u, w["gate"]) + lin(u, w["up"]), w["down"])
    heads = attn.shape[-1] // kv.shape[-1]
    return x + 0.05 * (attn + ffn + kv.repeat(1, heads))


class Block:
    """Layer ``index`` as a function of (x, gain) for ``checkpoint``.  The
    weights are materialised inside the call, i.e. inside the checkpointed
    region: a recompute that runs this far materialises them again."""

    def __init__(self, source: WeightSource, index: int, lin):
        self.source, self.index, self.lin = source, index, lin

    def __call__(self, x, gain):
        u = torch.mul(x, gain)
        return mix(x, u, self.source.weights(self.index), self.lin)


@dataclass
class Workload:
    packed: list                     # LayerBuffer per layer
    dense: list                      # DenseBlockStore per layer (may be empty)
    x: torch.Tensor                  # [tokens, width] bf16 input
    gains: list                      # initial gain vector per layer
    probe: torch.Tensor              # [tokens, width] fp32 output projection


@dataclass
class StepResult:
    loss: torch.Tensor
    grads: List[torch.Tensor] = field(default_factory=list)   # one per gain, then the input's


def make_workload(layers: int = 8, tokens: int = 256, projs=WL.QWEN_32B, seed: int = 0,
                  dense: bool = True, device="cuda") -> Workload:
    """Seeded synthetic layers: weights 0.02 N(0,1) quantised to nested NF4
    on the device; the dense control holds the dequantised W_hat of the same
    weights, so both arms multiply by identical values."""
    dev = torch.device(device)
    code = torch.from_numpy(WL.nf4_code_np()).to(dev)
    ncode = torch.from_numpy(WL.nested_code_np()).to(dev)
    names = [p.name for p in projs]
    packed, dense_stores = [], []
    for l in range(layers):
        qs = []
        for i, p in enumerate(projs):
            w = WL.gpu_weight_f32(p.N, p.K, seed=80_000 + 100 * seed + 16 * l + i, device=dev)
            qs.append(api.nf4_quantize(w, code, ncode))
            del w
        packed.append(LayerBuffer(names, qs))
        if dense:
            dense_stores.append(DenseBlockStore(names, [api.nf4_dequantize(q) for q in qs]))
        del qs
    width = projs[0].K
    x = WL.gpu_normal_bf16(tokens, width, seed=81_000 + seed, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(82_000 + seed)
    gains = [(1.0 + 0.01 * torch.randn(width, generator=gen, device=dev)).to(torch.bfloat16)
             for _ in range(layers)]
    probe = torch.randn((tokens, width), generator=gen, device=dev) / tokens
    torch.cuda.synchronize()
    return Workload(packed, dense_stores, x, gains, probe)


def train_step(work: Workload, arm: str, reuse: bool, slots: int = 2, checkpointed: bool = True,
               early_stop: bool = True) -> StepResult:
    """Forward through every block, then the backward of <probe, output>.

    With early stop (torch's default) a block's recompute ends once the
    tensors its forward saved are rebuilt.  For the negative control that
    happens before the weights are materialised again, so the slots keep
    their forward contents and the last ``slots`` layers come out right.
    Without early stop every recompute refills a slot before the ctx-held
    backward reads it, and only the last layer is right."""
    stores = work.dense if arm == "dense" else work.packed
    source = WeightSource(stores, reuse, slots)
    lin = projection(arm)
    gains = [g.clone().requires_grad_(True) for g in work.gains]
    x_in = work.x.clone().requires_grad_(True)
    act = x_in
    for index, gain in enumerate(gains):
        block = Block(source, index, lin)
        if checkpointed:
            act = checkpoint(block, act, gain, use_reentrant=False, early_stop=early_stop)
        else:
            act = block(act, gain)
    objective = torch.sum(act.float() * work.probe)
    objective.backward()
    torch.cuda.synchronize()
    grads = [g.grad.detach().clone() for g in gains] + [x_in.grad.detach().clone()]
    return StepResult(objective.detach().clone(), grads)


def grad_gaps(a: StepResult, b: StepResult) -> List[float]:
    """max |a - b| per gradient (the gains in layer order, then the input)."""
    return [float(torch.max(torch.abs(u.float() - v.float())).item()) for u, v in zip(a.grads, b.grads)]


def compare_arms(work: Workload, slots: int = 2) -> Dict[str, dict]:
    """Per arm: whether the loss is bit-equal between reused and private
    buffers, and the per-gradient gaps between the two."""
    out = {}
    for arm in ARMS:
        if arm == "dense" and not work.dense:
            continue
        private = train_step(work, arm, reuse=False, slots=slots)
        reused = train_step(work, arm, reuse=True, slots=slots)
        out[arm] = {"loss_equal": bool(torch.equal(private.loss, reused.loss)),
                    "gaps": grad_gaps(reused, private)}
    return out


def main(argv) -> int:
    slots = int(argv[0]) if argv else 2
    work = make_workload()
    res = compare_arms(work, slots)
    n = len(work.packed)
    print(f"{n} layers of {work.packed[0].nbytes / 2 ** 20:.1f} MiB nested NF4 through {slots} reused slots")
    for arm, r in res.items():
        exact = [i for i, g in enumerate(r["gaps"][:n]) if g == 0.0]
        worst = max(r["gaps"])
        print(f"  {arm:>9}: loss bit-equal {r['loss_equal']}; layers with exact gain gradients "
              f"{exact or 'none'}; input gradient gap {r['gaps'][n]:.3e}; largest gap {worst:.3e}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
