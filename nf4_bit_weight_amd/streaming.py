"""Layer streaming: NF4 layers kept in page-locked host memory and copied into
a small ring of device slots on every visit.

Soup issue #842 ("Why", "Acceptance criteria") describes the caller this
serves: each streamed layer's packed weights are copied host-to-device into
pooled buffers on every visit, the forward walks the layers in order and the
backward walks them in reverse, so every layer is copied twice per step and
device memory holds only the ring.  Because the fused kernels read the
packed fields directly, nothing dense is written per visit; streamed and
resident weights go through the same kernels on the same bytes, so their
outputs are bit-identical.

Plumbing only (torch streams, events and copies; no arithmetic):

* ``LayerBuffer`` lays out the NF4 fields (packed, absmax, nested absmax,
  nested offset) of a layer's projections in one byte buffer, every field
  256-byte aligned, so one copy moves a layer; ``views(buf)`` rebuilds the
  ``NF4Weight`` of each projection on any buffer of that layout.
* ``SlotStreamer`` runs a list of layer visits: visit v uses slot v % S; the
  copy for visit v + S - 1 is issued on a separate copy stream (default
  priority) once the compute that last used its slot has been enqueued, and
  the compute stream waits on the copy's event before the visit's kernels.
  A run's first copies wait for everything already on the compute stream,
  so consecutive runs never overwrite a slot still being read.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence

import torch

from .api import NF4Weight

ALIGN = 256


def _round_up(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


@dataclass
class _Field:
    offset: int
    numel: int
    dtype: torch.dtype
    itemsize: int


class LayerBuffer:
    """One layer's NF4 fields in a single byte buffer (see module doc).  The
    code tables stay outside: they are the same for every layer."""

    def __init__(self, names: Sequence[str], weights: Sequence[NF4Weight], pin_memory: bool = False,
                 device: Optional[torch.device] = None):
        if len(names) != len(weights) or not weights:
            raise ValueError("one name per weight, at least one weight")
        self.names = list(names)
        self.spec = []
        off = 0
        for w in weights:
            fields = []
            for t in w.tensors()[:4]:
                if t is None:
                    fields.append(None)
                    continue
                fields.append(_Field(off, t.numel(), t.dtype, t.element_size()))
                off += _round_up(t.numel() * t.element_size())
            self.spec.append((fields, w.N, w.K))
        self.nbytes = off
        self.code, self.nested_code = weights[0].code, weights[0].nested_code
        dev = weights[0].packed.device if device is None else device
        # zero-filled, so the alignment padding is the same in every copy
        if pin_memory:
            self.store = torch.zeros(off, dtype=torch.uint8, pin_memory=True)
        else:
            self.store = torch.zeros(off, dtype=torch.uint8, device=dev)
        for w, (fields, _, _) in zip(weights, self.spec):
            for t, f in zip(w.tensors()[:4], fields):
                if f is not None:
                    n = f.numel * f.itemsize
                    self.store[f.offset:f.offset + n].copy_(t.reshape(-1).view(torch.uint8))

    def views(self, buf: torch.Tensor) -> dict:
        """{name: NF4Weight} whose fields are views into ``buf``, a buffer of
        this layout (the store itself, or a device slot)."""
        if buf.dtype != torch.uint8 or buf.numel() < self.nbytes:
            raise ValueError(f"buffer must be uint8 with at least {self.nbytes} bytes")
        out = {}
        for name, (fields, N, K) in zip(self.names, self.spec):
            ts = [None if f is None else buf[f.offset:f.offset + f.numel * f.itemsize].view(f.dtype)
                  for f in fields]
            out[name] = NF4Weight(ts[0], ts[1], ts[2], ts[3], self.code, self.nested_code, N, K)
        return out


class SlotStreamer:
    """Streams layers from host buffers through ``n_slots`` device slots."""

    def __init__(self, host_layers: Sequence[LayerBuffer], n_slots: int, device):
        if n_slots < 2:
            raise ValueError("at least two slots: one computing, one filling")
        self.layers = list(host_layers)
        nbytes = max(l.nbytes for l in self.layers)
        self.slots = [torch.empty(nbytes, dtype=torch.uint8, device=device) for _ in range(n_slots)]
        self.copy_stream = torch.cuda.Stream(device=device)
        self.ready = [torch.cuda.Event() for _ in range(n_slots)]
        self.free = [torch.cuda.Event() for _ in range(n_slots)]
        self.bytes_copied = 0

    @property
    def device_bytes(self) -> int:
        return sum(s.numel() for s in self.slots)

    def _issue(self, visits: List[int], v: int, compute: torch.cuda.Stream):
        s = v % len(self.slots)
        with torch.cuda.stream(self.copy_stream):
            if v >= len(self.slots):
                self.copy_stream.wait_event(self.free[s])     # the slot's last reader is enqueued
            src = self.layers[visits[v]].store
            self.slots[s][:src.numel()].copy_(src, non_blocking=True)
            self.ready[s].record(self.copy_stream)
        self.bytes_copied += self.layers[visits[v]].nbytes

    def run(self, visits: Sequence[int], fn: Callable[[int, int, dict], None]) -> None:
        """For each visit v (a layer index), wait for its slot to be filled
        and call fn(v, layer, weights) with the layer's weights viewed in the
        slot; fn enqueues its kernels on the current stream."""
        visits = list(visits)
        compute = torch.cuda.current_stream()
        S = len(self.slots)
        # every slot may still be read by work already on the compute stream
        # (an earlier run): no copy starts before that work
        self.copy_stream.wait_stream(compute)
        for v in range(min(S - 1, len(visits))):
            self._issue(visits, v, compute)
        for v, layer in enumerate(visits):
            if v + S - 1 < len(visits):
                self._issue(visits, v + S - 1, compute)
            s = v % S
            compute.wait_event(self.ready[s])
            fn(v, layer, self.layers[layer].views(self.slots[s]))
            self.free[s].record(compute)
