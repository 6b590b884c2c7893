"""Uploads logical weight arrays (numpy, storage dtypes) to device memory and
packs expert bundles into a slot pool with edge0_pack_bundle.  Data movement
only."""
from __future__ import annotations

import numpy as np
import torch

from . import edge0 as E


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy array in a storage dtype -> torch device tensor with the same bytes."""
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to(device)


def bf16_tensor_to_numpy(t: torch.Tensor) -> np.ndarray:
    """int16 device tensor of bf16 bits -> numpy uint16."""
    return t.detach().cpu().numpy().view(np.uint16)


class SlotPoolBuffer:
    """Device memory for n_slots bundles and the SlotPool struct describing it."""

    def __init__(self, shape: E.MoeShape, n_slots: int, device="cuda"):
        self.shape = shape
        self.layout = E.edge0_bundle_layout_of(shape)
        self.slot_bytes = int(self.layout.bytes)
        self.n_slots = n_slots
        self.mem = torch.zeros(n_slots * self.slot_bytes, dtype=torch.uint8, device=device)
        self.pool = E.SlotPool(self.mem.data_ptr(), self.slot_bytes, n_slots)

    def slot_ptr(self, s: int) -> int:
        return self.mem.data_ptr() + s * self.slot_bytes

    def load(self, s: int, expert: dict, lora: dict | None = None, stream=None):
        """Pack one expert (and its LoRA) from logical numpy arrays into slot s."""
        arrays = {k: to_device(v) for k, v in expert.items()}
        if lora is not None:
            arrays.update({k: to_device(v) for k, v in lora.items()})
        E.edge0_pack_bundle(self.shape, arrays, self.slot_ptr(s), stream)
        torch.cuda.current_stream().synchronize()

    def bundle_bytes(self, s: int) -> torch.Tensor:
        return self.mem[s * self.slot_bytes:(s + 1) * self.slot_bytes]


def head_to_device(head: dict) -> dict:
    return {k: (None if v is None else to_device(v)) for k, v in head.items()}
