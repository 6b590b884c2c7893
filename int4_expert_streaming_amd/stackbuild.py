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
                 threads=16, log=print, separate_lora=False):
        """separate_lora: LoRA-free bundles in the pool and each layer's
        adapters in a device block of their own, one per expert
        (edge0_stack_create_lora)."""
        self.S = shape
        self.sh = E.make_shape(shape)
        En = shape.n_experts
        self.n_layers = n_layers
        self.spec = E.StackSpec(n_layers, owners[0], owners[1], consumers[0], consumers[1], eps)
        self.owners = range(owners[0], owners[1] + 1)
        self.consumers = range(consumers[0], consumers[1] + 1)
        sep = separate_lora and shape.lora_rank > 0
        self.sh_pool = E.make_shape(shape)
        if sep:
            self.sh_pool.lora_rank = 0  # the bundles hold the int4 arrays only
        self.pool = SlotPoolBuffer(self.sh_pool, n_layers * En)
        self.lora_blocks, self.loras = [], None
        t0 = time.time()
        with ThreadPoolExecutor(threads) as ex:
            for L in range(n_layers):
                parts = list(ex.map(lambda e: (gen.expert(L, e), gen.lora(L, e)), range(En)))
                if sep:
                    lo, block = lora_block([p[1] for p in parts])
                    self.lora_blocks.append(block)
                    self.loras = (self.loras or []) + [lo]
                    parts = [(p[0], None) for p in parts]
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
                             self.heads, loras=self.loras)
        if log:
            log(f"[stack] ready: {n_layers} layers, pool {self.pool.mem.numel() / 1e9:.2f} GB "
                f"({time.time() - t0:.1f}s)")

    def _pack_layer(self, L, parts):
        En = self.S.n_experts
        pack_layer(self.sh_pool, parts, lambda e: self.pool.slot_ptr(L * En + e))

    def step(self, h0, h_out, step):
        self.stack.step(h0, h_out, step)


LORA_FACTORS = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def lora_block(loras):
    """One layer's adapters (loras[e] = the six bf16 factor arrays of expert
    e) as one device block, [E][a_gate|b_gate|a_up|b_up|a_down|b_down], and
    the Lora struct pointing at expert 0's factors with a stride of one
    expert's block."""
    rows = [np.concatenate([np.asarray(lo[f]).ravel() for f in LORA_FACTORS]) for lo in loras]
    block = to_device(np.ascontiguousarray(np.stack(rows)).view(np.uint16))
    offs = np.cumsum([0] + [np.asarray(loras[0][f]).size for f in LORA_FACTORS])
    base = block.data_ptr()
    return E.Lora(*[base + 2 * int(offs[i]) for i in range(6)], rows[0].size), block


def pack_layer(sh, parts, dst_of):
    """Packs one layer's experts (parts[e] = (expert arrays, lora arrays))
    into the device bundles at dst_of(e)."""
    keys = list(parts[0][0].keys()) + (list(parts[0][1].keys()) if parts[0][1] else [])
    stacked = {}
    for k in keys:
        src = [p[0][k] if k in p[0] else p[1][k] for p in parts]
        stacked[k] = to_device(np.stack(src))
    for e in range(len(parts)):
        E.edge0_pack_bundle(sh, {k: v[e] for k, v in stacked.items()}, dst_of(e))
    torch.cuda.synchronize()


class HostBundles:
    """Every (layer, expert) bundle in the device bundle layout, in pinned
    host memory (the source tier of the staged pool): packed on the device
    one layer at a time and copied back."""

    def __init__(self, shape, gen, n_layers, threads=16, log=print):
        self.sh = E.make_shape(shape)
        En = shape.n_experts
        self.bundle_bytes = int(E.edge0_bundle_layout_of(self.sh).bytes)
        bb = self.bundle_bytes
        self.mem = torch.empty(n_layers * En * bb, dtype=torch.uint8, pin_memory=True)
        tmp = SlotPoolBuffer(self.sh, En)
        t0 = time.time()
        with ThreadPoolExecutor(threads) as ex:
            for L in range(n_layers):
                parts = list(ex.map(lambda e: (gen.expert(L, e), gen.lora(L, e)), range(En)))
                pack_layer(self.sh, parts, tmp.slot_ptr)
                self.mem[L * En * bb:(L + 1) * En * bb].copy_(tmp.mem[:En * bb])
                if log and (L % 8 == 7 or L == n_layers - 1):
                    log(f"[host] packed layer {L + 1}/{n_layers} ({time.time() - t0:.1f}s)")
        del tmp
        base = self.mem.data_ptr()
        self.ptrs = [base + k * bb for k in range(n_layers * En)]

    def bundle(self, L, e, n_experts):
        k = L * n_experts + e
        return self.mem[k * self.bundle_bytes:(k + 1) * self.bundle_bytes]


def write_layer_files(host: "HostBundles", directory: str, n_experts: int, log=None):
    """Writes every layer of the host tier to its expert file under
    `directory` (layer_NNN.e0l); returns the paths in layer order."""
    import os
    os.makedirs(directory, exist_ok=True)
    n_layers = len(host.ptrs) // n_experts
    paths = []
    t0 = time.time()
    for L in range(n_layers):
        path = os.path.join(directory, f"layer_{L:03d}.e0l")
        E.layer_file_write(path, host.sh, L, host.ptrs[L * n_experts:(L + 1) * n_experts])
        paths.append(path)
    if log:
        log(f"[files] {n_layers} layer files written to {directory} ({time.time() - t0:.1f}s)")
    return paths


def device_routers_heads(gen, n_layers, owners, threads=16):
    """Device copies of every layer's router and of the owner layers' heads
    (None elsewhere)."""
    with ThreadPoolExecutor(threads) as ex:
        routers = list(ex.map(gen.router, range(n_layers)))
        heads = list(ex.map(lambda L: gen.head(L) if L in owners else None, range(n_layers)))
    return ([to_device(r) for r in routers],
            [None if h is None else head_to_device(h) for h in heads])


class StreamedStack:
    """The decode stack over a bounded HBM pool of n_slots slots, staged from
    pinned host bundles by the library's stager, routed by a given trace."""

    def __init__(self, shape, gen, n_layers, owners, consumers, n_slots, eps=1e-6, threads=16,
                 log=print, host=None, routers=None, heads=None, files=None):
        self.S = shape
        self.sh = E.make_shape(shape)
        En = shape.n_experts
        self.n_layers = n_layers
        self.spec = E.StackSpec(n_layers, owners[0], owners[1], consumers[0], consumers[1], eps)
        self.owners = range(owners[0], owners[1] + 1)
        self.consumers = range(consumers[0], consumers[1] + 1)
        # bundles come from the pinned host tier, or from a FileTier's layer files
        self.files = files
        self.host = host if (host is not None or files is not None) else \
            HostBundles(shape, gen, n_layers, threads, log)
        self.pool = SlotPoolBuffer(self.sh, n_slots)
        self.table = torch.full((n_layers, En), -1, dtype=torch.int32, device="cuda")
        if routers is None or heads is None:  # device copies, or built here
            routers, heads = device_routers_heads(gen, n_layers, self.owners, threads)
        self.routers, self.heads = routers, heads
        torch.cuda.synchronize()
        self.stack = E.Stack(self.sh, self.spec, self.pool.pool, self.table, self.routers,
                             self.heads)
        self.stager = E.Stager(self.sh, self.pool.pool, n_layers,
                               None if files is not None else self.host.ptrs, self.table, files)
        self.copy_stream = torch.cuda.Stream()

    def step(self, h0, h_out, step, ids_dev, ids_host, next_ids_host, ahead=True):
        E.stack_step_staged(self.stack, self.stager, h0, h_out, step, ids_dev, ids_host,
                            next_ids_host, ahead, self.copy_stream)
