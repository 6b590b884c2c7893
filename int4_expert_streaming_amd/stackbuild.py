"""Builds a decode stack on the device: every layer's experts packed into a
slot pool (slot = layer * E + expert), routers and heads uploaded, and the
edge0_stack handle created.  Weight values come from caller-supplied
generator callables; this module only moves bytes and calls the library."""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import edge0 as E
from .weights import SlotPoolBuffer, head_to_device, to_device


class DeviceStack:
    """gen must provide expert(L, e) -> dict of the nine logical arrays,
    lora(L, e) -> dict of the six adapter arrays (or None), router(L) ->
    bf16 bits [E][d], head(L) -> dict of fp16 head arrays."""

    def __init__(self, shape, gen, n_layers=40, owners=(6, 37), consumers=(7, 38), eps=1e-6,
                 threads=16, log=print):
        self.S = shape
        self.sh = E.make_shape(shape)
        En = shape.n_experts
        self.n_layers = n_layers
        self.spec = E.StackSpec(n_layers, owners[0], owners[1], consumers[0], consumers[1], eps)
        self.owners = range(owners[0], owners[1] + 1)
        self.consumers = range(consumers[0], consumers[1] + 1)
        self.pool = SlotPoolBuffer(self.sh, n_layers * En)
        t0 = time.time()
        with ThreadPoolExecutor(threads) as ex:
            for L in range(n_layers):
                parts = list(ex.map(lambda e: (gen.expert(L, e), gen.lora(L, e)), range(En)))
                self._pack_layer(L, parts)
                if log and (L % 8 == 7 or L == n_layers - 1):
                    log(f"[stack] packed layer {L + 1}/{n_layers} ({time.time() - t0:.1f}s)")
            routers = list(ex.map(gen.router, range(n_layers)))
            heads = list(ex.map(lambda L: gen.head(L) if L in self.owners else None,
                                range(n_layers)))
        self.routers = [to_device(r) for r in routers]
        self.heads = [None if h is None else head_to_device(h) for h in heads]
        self.tables = torch.arange(n_layers * En, dtype=torch.int32, device="cuda").view(n_layers, En)
        torch.cuda.synchronize()
        self.stack = E.Stack(self.sh, self.spec, self.pool.pool, self.tables, self.routers,
                             self.heads)
        if log:
            log(f"[stack] ready: {n_layers} layers, pool {self.pool.mem.numel() / 1e9:.2f} GB "
                f"({time.time() - t0:.1f}s)")

    def _pack_layer(self, L, parts):
        En = self.S.n_experts
        keys = list(parts[0][0].keys()) + (list(parts[0][1].keys()) if parts[0][1] else [])
        stacked = {}
        for k in keys:
            src = [p[0][k] if k in p[0] else p[1][k] for p in parts]
            stacked[k] = to_device(np.stack(src))
        for e in range(En):
            E.edge0_pack_bundle(self.sh, {k: v[e] for k, v in stacked.items()},
                                self.pool.slot_ptr(L * En + e))
        torch.cuda.synchronize()
        del stacked

    def step(self, h0, h_out, step):
        self.stack.step(h0, h_out, step)
