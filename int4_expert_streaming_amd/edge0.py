"""Thin ctypes binding of libedge0.so (the C ABI declared in include/edge0.h).

Argument marshalling only: torch tensors supply device pointers, the current
torch stream supplies the HIP stream, and every computation runs in the
library's HIP kernels.  Importing this module loads the library and fails
loudly if it has not been built.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os
import weakref

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libedge0.so")

EDGE0_OK, EDGE0_EINVAL, EDGE0_EHIP, EDGE0_ENOSLOT, EDGE0_ERANGE, EDGE0_ENOMEM = 0, -1, -2, -3, -4, -5
EDGE0_ESCRATCH = -6
EDGE0_ROUTE_SOFTMAX_TOPK = 0
EDGE0_STAGE_LOOP = 2
EDGE0_ROUTE_SIGMOID_GROUP = 1
EDGE0_STATIC_WORKSPACE_BYTES = 1 << 20


class Edge0Error(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    return C.CDLL(LIB_PATH)


lib = _load()

# Handles still open at interpreter exit are closed by an exit hook that runs
# before torch's own (hooks run last-registered first, and this module is
# imported after torch): each destroy call synchronises the device first,
# so no launch of a handle outlives its events, graphs or buffers, and no
# destroy runs from a finaliser after the HIP runtime has shut down.
_live = weakref.WeakSet()


@atexit.register
def _close_live_handles():
    for h in sorted(list(_live), key=lambda h: 0 if isinstance(h, Stager) else 1):
        try:
            h.close()
        except Exception:
            pass


class _Handle:
    """Context-manager and exit-hook behaviour of the opaque handles."""

    def _register(self):
        _live.add(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------------------------------- structs
class MoeShape(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_experts", C.c_int32), ("d_inter", C.c_int32),
                ("top_k", C.c_int32), ("group_size", C.c_int32), ("lora_rank", C.c_int32),
                ("lora_alpha", C.c_float), ("head_hidden", C.c_int32), ("routing", C.c_int32),
                ("n_groups", C.c_int32), ("top_groups", C.c_int32), ("route_scale", C.c_float)]


_LAYOUT_KEYS = ("gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b", "down_q", "down_s",
                "down_b", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


class BundleLayout(C.Structure):
    _fields_ = [(k, C.c_int64) for k in _LAYOUT_KEYS] + [("bytes", C.c_int64)]


class ExpertArrays(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in _LAYOUT_KEYS]


class SlotPool(C.Structure):
    _fields_ = [("base", C.c_void_p), ("slot_bytes", C.c_int64), ("n_slots", C.c_int32)]


_HEAD_KEYS = ("w1x", "w1oh", "b1", "w2", "b2", "wl")


class Head(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in _HEAD_KEYS]


class StackSpec(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("owner_first", C.c_int32), ("owner_last", C.c_int32),
                ("consumer_first", C.c_int32), ("consumer_last", C.c_int32),
                ("rms_eps", C.c_float)]


class StackBuffers(C.Structure):
    _fields_ = [("x", C.c_void_p), ("y", C.c_void_p), ("h", C.c_void_p), ("ids", C.c_void_p),
                ("w", C.c_void_p), ("pred_ids", C.c_void_p), ("pred_w", C.c_void_p)]


class StageStats(C.Structure):
    _fields_ = [("requests", C.c_int64), ("touches", C.c_int64), ("hits", C.c_int64),
                ("misses", C.c_int64), ("evictions", C.c_int64), ("bytes_staged", C.c_int64)]


class StagePlan(C.Structure):
    _fields_ = [("ids_dev", C.c_void_p), ("ids_host", C.c_void_p), ("next_ids_host", C.c_void_p),
                ("ahead", C.c_int32), ("copy_stream", C.c_void_p)]


_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)
_SIG = {
    "edge0_strerror": (C.c_char_p, [C.c_int]),
    "edge0_bundle_layout_of": (C.c_int, [C.POINTER(MoeShape), C.POINTER(BundleLayout)]),
    "edge0_pack_bundle": (C.c_int, [C.POINTER(MoeShape), C.POINTER(ExpertArrays), _P, _P]),
    "edge0_workspace_bytes": (C.c_size_t, [C.POINTER(MoeShape)]),
    "edge0_workspace_error": (C.c_int, [_P, _P]),
    "edge0_route_commit": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P]),
    "edge0_moe_layer_lora": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, _P, _P, _P,
                                       _P, _P, _P, _P]),
    "edge0_prefill_workspace_bytes": (C.c_size_t, [C.POINTER(MoeShape), C.c_int32]),
    "edge0_merge_workspace_bytes": (C.c_size_t, [C.POINTER(MoeShape)]),
    "edge0_merge_requant": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P]),
    "edge0_moe_prefill": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, C.c_int32, _P,
                                    _P, _P, _P, _P, C.c_int32, _P]),
    "edge0_router": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, _P, _P]),
    "edge0_prerouter": (C.c_int, [C.POINTER(MoeShape), C.POINTER(Head), _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P]),
    "edge0_stack_set_trace": (C.c_int, [_P, C.c_int32, _P]),
    "edge0_moe_layer_noalloc": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, _P, _P,
                                          _P, _P, _P, _P]),
    "edge0_moe_layer": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, _P, _P, _P, _P,
                                  _P, _P]),
    "edge0_stack_create": (C.c_int, [C.POINTER(_P), C.POINTER(MoeShape), C.POINTER(StackSpec),
                                     C.POINTER(SlotPool), _P, C.POINTER(_P), C.POINTER(Head)]),
    "edge0_stack_create_lora": (C.c_int, [C.POINTER(_P), C.POINTER(MoeShape), C.POINTER(StackSpec),
                                          C.POINTER(SlotPool), _P, C.POINTER(_P), C.POINTER(Head),
                                          _P]),
    "edge0_stack_step": (C.c_int, [_P, _P, _P, C.c_int32, _P]),
    "edge0_stack_get_buffers": (C.c_int, [_P, C.POINTER(StackBuffers)]),
    "edge0_stack_destroy": (None, [_P]),
    "edge0_stack_set_timing": (C.c_int, [_P, C.c_int32]),
    "edge0_stack_set_mode": (C.c_int, [_P, C.c_int32]),
    "edge0_stack_set_head_schedule": (C.c_int, [_P, C.c_int32]),
    "edge0_stack_set_spin_limit": (C.c_int, [_P, C.c_int64]),
    "edge0_stack_error": (C.c_int, [_P]),
    "edge0_stack_kernel_ms": (C.c_int, [_P, C.POINTER(C.c_float), C.c_int32,
                                        C.POINTER(C.c_int32)]),
    "edge0_stack_step_staged": (C.c_int, [_P, _P, C.POINTER(StagePlan), _P, _P, C.c_int32, _P]),
    "edge0_grouped_workspace_bytes": (C.c_size_t, [C.POINTER(MoeShape)]),
    "edge0_moe_grouped": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, C.c_int32, _P,
                                    _P, _P, _P, _P, C.c_int32, _P]),
    "edge0_moe_grouped_lora": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, _P,
                                         C.c_int32, _P, _P, _P, _P, _P, C.c_int32, _P]),
    "edge0_moe_prefill_lora": (C.c_int, [C.POINTER(MoeShape), C.POINTER(SlotPool), _P, _P,
                                         C.c_int32, _P, _P, _P, _P, _P, C.c_int32, _P]),
    "edge0_lru_create": (C.c_int, [C.POINTER(_P), C.c_int32, C.c_int32, C.c_int32]),
    "edge0_lru_request": (C.c_int, [_P, C.c_int32, C.c_int32, _I32P, C.c_int32, _I32P, _I32P,
                                    _I32P]),
    "edge0_lru_release": (C.c_int, [_P, C.c_int32, C.c_int32]),
    "edge0_lru_stats": (C.c_int, [_P, C.POINTER(StageStats)]),
    "edge0_lru_destroy": (None, [_P]),
    "edge0_stager_create": (C.c_int, [C.POINTER(_P), C.POINTER(MoeShape), C.POINTER(SlotPool),
                                      C.c_int32, C.POINTER(_P), _P]),
    "edge0_stager_create_files": (C.c_int, [C.POINTER(_P), C.POINTER(MoeShape),
                                            C.POINTER(SlotPool), C.c_int32, _P, _P]),
    "edge0_layer_file_record_bytes": (C.c_int64, [C.POINTER(MoeShape)]),
    "edge0_layer_file_write": (C.c_int, [C.c_char_p, C.POINTER(MoeShape), C.c_int32,
                                         C.POINTER(_P)]),
    "edge0_filetier_create": (C.c_int, [C.POINTER(_P), C.POINTER(MoeShape), C.c_int32,
                                        C.POINTER(C.c_char_p), C.c_int32, C.c_int32, C.c_int32]),
    "edge0_filetier_stats": (C.c_int, [_P, _P]),
    "edge0_filetier_destroy": (None, [_P]),
    "edge0_stage_experts": (C.c_int, [_P, C.c_int32, C.c_int32, _I32P, C.c_int32, _I32P, _P]),
    "edge0_stager_wait": (C.c_int, [_P, C.c_int32, C.c_int32, _P]),
    "edge0_stager_release": (C.c_int, [_P, C.c_int32, C.c_int32, _P]),
    "edge0_stager_flush": (C.c_int, [_P, _P]),
    "edge0_stager_set_copy_mode": (C.c_int, [_P, C.c_int32]),
    "edge0_stager_stats": (C.c_int, [_P, C.POINTER(StageStats)]),
    "edge0_stager_destroy": (None, [_P]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def strerror(code: int) -> str:
    return lib.edge0_strerror(code).decode()


def _check(code: int, where: str):
    if code != EDGE0_OK:
        raise Edge0Error(code, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_shape(s, routing: int = 0, n_groups: int = 0, top_groups: int = 0,
               route_scale: float = 0.0) -> MoeShape:
    """MoeShape from any object with the MoE spec fields (d_model, n_experts,
    d_inter, top_k, group, lora_rank, lora_alpha, head_hidden), plus the
    routing family (EDGE0_ROUTE_*) and its sigmoid-group parameters."""
    return MoeShape(s.d_model, s.n_experts, s.d_inter, s.top_k, s.group, s.lora_rank,
                    float(s.lora_alpha), s.head_hidden, routing, n_groups, top_groups,
                    float(route_scale))


# --------------------------------------------------------------------- calls
def edge0_bundle_layout_of(shape: MoeShape) -> BundleLayout:
    lay = BundleLayout()
    _check(lib.edge0_bundle_layout_of(C.byref(shape), C.byref(lay)), "edge0_bundle_layout_of")
    return lay


def edge0_workspace_bytes(shape: MoeShape) -> int:
    n = lib.edge0_workspace_bytes(C.byref(shape))
    if n == 0:
        raise Edge0Error(EDGE0_EINVAL, "edge0_workspace_bytes")
    return int(n)


def new_workspace(shape: MoeShape, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of edge0_workspace_bytes(shape) bytes."""
    return torch.zeros(edge0_workspace_bytes(shape), dtype=torch.uint8, device=device)


def edge0_workspace_error(workspace, stream=None) -> int:
    return lib.edge0_workspace_error(_ptr(workspace), _stream(stream))


def edge0_pack_bundle(shape: MoeShape, arrays: dict, bundle_dst, stream=None):
    """arrays: name -> device tensor in the logical layout (see ExpertArrays)."""
    src = ExpertArrays(**{k: _ptr(arrays.get(k)) for k in _LAYOUT_KEYS})
    _check(lib.edge0_pack_bundle(C.byref(shape), C.byref(src), _ptr(bundle_dst), _stream(stream)),
           "edge0_pack_bundle")


def edge0_route_commit(shape: MoeShape, logits, ids_out, w_out, route_bias=None, stream=None):
    _check(lib.edge0_route_commit(C.byref(shape), _ptr(logits), _ptr(route_bias), _ptr(ids_out),
                                  _ptr(w_out), _stream(stream)), "edge0_route_commit")


def edge0_router(shape: MoeShape, w_router, x, logits_out, ids_out, w_out, workspace,
                 stream=None, route_bias=None):
    _check(lib.edge0_router(C.byref(shape), _ptr(w_router), _ptr(route_bias), _ptr(x),
                            _ptr(logits_out), _ptr(ids_out), _ptr(w_out), _ptr(workspace),
                            _stream(stream)), "edge0_router")


def make_head(tensors: dict) -> Head:
    return Head(**{k: _ptr(tensors.get(k)) for k in _HEAD_KEYS})


def edge0_prerouter(shape: MoeShape, head: Head, x, ids_now, ids_prev, logits_out, ids_out, w_out,
                    workspace, stream=None, route_bias=None):
    _check(lib.edge0_prerouter(C.byref(shape), C.byref(head), _ptr(route_bias), _ptr(x),
                               _ptr(ids_now),
                               _ptr(ids_prev), _ptr(logits_out), _ptr(ids_out), _ptr(w_out),
                               _ptr(workspace), _stream(stream)), "edge0_prerouter")


class Lora(C.Structure):
    """The six bf16 factors of expert 0 and the element stride to the next
    expert's (0: one adapter shared by every expert)."""
    _fields_ = [(k, C.c_void_p) for k in ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")] + \
        [("expert_stride", C.c_int64)]


def edge0_moe_layer_lora(shape: MoeShape, pool: SlotPool, lora: "Lora | None", slot_table, ids, w,
                         x, y, workspace, stream=None):
    _check(lib.edge0_moe_layer_lora(C.byref(shape), C.byref(pool),
                                    None if lora is None else C.byref(lora), _ptr(slot_table),
                                    _ptr(ids), _ptr(w), _ptr(x), _ptr(y), _ptr(workspace),
                                    _stream(stream)), "edge0_moe_layer_lora")


def edge0_moe_layer(shape: MoeShape, pool: SlotPool, slot_table, ids, w, x, y, workspace,
                    stream=None):
    _check(lib.edge0_moe_layer(C.byref(shape), C.byref(pool), _ptr(slot_table), _ptr(ids), _ptr(w),
                               _ptr(x), _ptr(y), _ptr(workspace), _stream(stream)),
           "edge0_moe_layer")


def edge0_moe_layer_noalloc(shape: MoeShape, pool: SlotPool, slot_table, ids, w, x, y,
                            error_out=None, stream=None):
    """edge0_moe_layer on the library's static per-GPU workspace."""
    _check(lib.edge0_moe_layer_noalloc(C.byref(shape), C.byref(pool), _ptr(slot_table), _ptr(ids),
                                       _ptr(w), _ptr(x), _ptr(y), _ptr(error_out), _stream(stream)),
           "edge0_moe_layer_noalloc")


EDGE0_GROUPED_NO_MFMA = 1
EDGE0_STACK_GRAPHS = 0
EDGE0_STACK_PERSISTENT = 1
EDGE0_STACK_XCD = 2
EDGE0_STACK_XLAYER = 3
EDGE0_HEADS_AFTER_LAYERS = 0
EDGE0_HEADS_FOLDED = 1


def grouped_mfma_min(n: int) -> int:
    """Flag putting the grouped layer's experts with >= n tokens on MFMA."""
    return (n & 0xFF) << 8


def new_grouped_workspace(shape: MoeShape, device="cuda") -> torch.Tensor:
    """Zero-filled workspace for edge0_moe_grouped."""
    n = lib.edge0_grouped_workspace_bytes(C.byref(shape))
    if n == 0:
        raise Edge0Error(EDGE0_EINVAL, "edge0_grouped_workspace_bytes")
    return torch.zeros(int(n), dtype=torch.uint8, device=device)


def edge0_merge_requant(shape: MoeShape, src_bundle, dst_bundle, stats_out, workspace=None,
                        stream=None):
    """Merges one expert's LoRA into its int4 weights (edge0_merge_requant);
    stats_out: device float64 [6]."""
    if workspace is None:
        workspace = torch.empty(lib.edge0_merge_workspace_bytes(C.byref(shape)), dtype=torch.uint8,
                                device="cuda")
    _check(lib.edge0_merge_requant(C.byref(shape), _ptr(src_bundle), _ptr(dst_bundle),
                                   _ptr(stats_out), _ptr(workspace), _stream(stream)),
           "edge0_merge_requant")
    return workspace


def new_prefill_workspace(shape: MoeShape, max_tokens: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace for edge0_moe_prefill calls of up to max_tokens."""
    n = lib.edge0_prefill_workspace_bytes(C.byref(shape), max_tokens)
    if n == 0:
        raise Edge0Error(EDGE0_EINVAL, "edge0_prefill_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def edge0_moe_prefill(shape: MoeShape, pool: SlotPool, slot_table, n_tokens: int, ids, w, x, y,
                      workspace, max_tokens: int, stream=None):
    _check(lib.edge0_moe_prefill(C.byref(shape), C.byref(pool), _ptr(slot_table), n_tokens,
                                 _ptr(ids), _ptr(w), _ptr(x), _ptr(y), _ptr(workspace), max_tokens,
                                 _stream(stream)), "edge0_moe_prefill")


def edge0_moe_grouped(shape: MoeShape, pool: SlotPool, slot_table, n_tokens: int, ids, w, x, y,
                      workspace, flags: int = 0, stream=None):
    _check(lib.edge0_moe_grouped(C.byref(shape), C.byref(pool), _ptr(slot_table), n_tokens,
                                 _ptr(ids), _ptr(w), _ptr(x), _ptr(y), _ptr(workspace), flags,
                                 _stream(stream)), "edge0_moe_grouped")


def edge0_moe_grouped_lora(shape: MoeShape, pool: SlotPool, lora: "Lora | None", slot_table,
                           n_tokens: int, ids, w, x, y, workspace, flags: int = 0, stream=None):
    _check(lib.edge0_moe_grouped_lora(C.byref(shape), C.byref(pool),
                                      None if lora is None else C.byref(lora), _ptr(slot_table),
                                      n_tokens, _ptr(ids), _ptr(w), _ptr(x), _ptr(y),
                                      _ptr(workspace), flags, _stream(stream)),
           "edge0_moe_grouped_lora")


def edge0_moe_prefill_lora(shape: MoeShape, pool: SlotPool, lora: "Lora | None", slot_table,
                           n_tokens: int, ids, w, x, y, workspace, max_tokens: int, stream=None):
    _check(lib.edge0_moe_prefill_lora(C.byref(shape), C.byref(pool),
                                      None if lora is None else C.byref(lora), _ptr(slot_table),
                                      n_tokens, _ptr(ids), _ptr(w), _ptr(x), _ptr(y),
                                      _ptr(workspace), max_tokens, _stream(stream)),
           "edge0_moe_prefill_lora")


class Stack(_Handle):
    """Owner of an edge0_stack handle (decode stack runtime)."""

    def __init__(self, shape: MoeShape, spec: StackSpec, pool: SlotPool, slot_tables, routers,
                 heads, loras=None):
        """loras: None (adapters in the bundles) or one Lora per layer
        (edge0_stack_create_lora)."""
        self.shape, self.spec = shape, spec
        self._keep = (slot_tables, routers, heads, loras)
        n = spec.n_layers
        router_ptrs = (C.c_void_p * n)(*[_ptr(r) for r in routers])
        head_arr = (Head * n)(*[make_head(h) if h is not None else Head() for h in heads])
        self._handle = C.c_void_p()
        if loras is None:
            _check(lib.edge0_stack_create(C.byref(self._handle), C.byref(shape), C.byref(spec),
                                          C.byref(pool), _ptr(slot_tables), router_ptrs, head_arr),
                   "edge0_stack_create")
        else:
            lora_arr = (Lora * n)(*loras)
            self._keep = self._keep + (lora_arr,)
            _check(lib.edge0_stack_create_lora(C.byref(self._handle), C.byref(shape), C.byref(spec),
                                               C.byref(pool), _ptr(slot_tables), router_ptrs,
                                               head_arr, C.cast(lora_arr, C.c_void_p)),
                   "edge0_stack_create_lora")
        self._register()

    def step(self, h0, h_out, step: int, stream=None):
        _check(lib.edge0_stack_step(self._handle, _ptr(h0), _ptr(h_out), step, _stream(stream)),
               "edge0_stack_step")

    def set_mode(self, mode: int):
        """EDGE0_STACK_GRAPHS (per-layer launches as graphs) or
        EDGE0_STACK_PERSISTENT (one cooperative launch for the layers)."""
        _check(lib.edge0_stack_set_mode(self._handle, mode), "edge0_stack_set_mode")

    def set_head_schedule(self, schedule: int):
        """EDGE0_HEADS_FOLDED (heads beside the down launches) or
        EDGE0_HEADS_AFTER_LAYERS (one batch after the last layer)."""
        _check(lib.edge0_stack_set_head_schedule(self._handle, schedule),
               "edge0_stack_set_head_schedule")

    def set_spin_limit(self, polls: int):
        _check(lib.edge0_stack_set_spin_limit(self._handle, polls), "edge0_stack_set_spin_limit")

    def error(self) -> int:
        """The handle's recorded error code (EDGE0_OK, EDGE0_ERANGE, EDGE0_EHIP), cleared."""
        return int(lib.edge0_stack_error(self._handle))

    def set_timing(self, kernel: int):
        """Event pair around one launch class per layer (1 gate/up, 2 down, 3 LoRA-in)."""
        _check(lib.edge0_stack_set_timing(self._handle, kernel), "edge0_stack_set_timing")

    def set_trace(self, layer: int, buf=None):
        """XCD mode: per-workgroup clock stamps of one layer into buf (int64 [256][16])."""
        _check(lib.edge0_stack_set_trace(self._handle, layer, _ptr(buf)), "edge0_stack_set_trace")

    def kernel_ms(self) -> list:
        n = self.spec.n_layers
        out = (C.c_float * n)()
        cnt = C.c_int32()
        _check(lib.edge0_stack_kernel_ms(self._handle, out, n, C.byref(cnt)), "edge0_stack_kernel_ms")
        return list(out[:cnt.value])

    def buffers(self) -> dict:
        """Views of the handle's per-layer device buffers from the last step."""
        b = StackBuffers()
        _check(lib.edge0_stack_get_buffers(self._handle, C.byref(b)), "edge0_stack_get_buffers")
        n, d, K = self.spec.n_layers, self.shape.d_model, self.shape.top_k
        return {
            "x": _wrap(b.x, (n, d), torch.int16), "y": _wrap(b.y, (n, d), torch.int16),
            "h": _wrap(b.h, (n + 1, d), torch.int16), "ids": _wrap(b.ids, (n, K), torch.int32),
            "w": _wrap(b.w, (n, K), torch.float32),
            "pred_ids": _wrap(b.pred_ids, (n, K), torch.int32),
            "pred_w": _wrap(b.pred_w, (n, K), torch.float32),
        }

    def close(self):
        if self._handle:
            lib.edge0_stack_destroy(self._handle)
            self._handle = C.c_void_p()



def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _stats(s: StageStats) -> dict:
    return {k: int(getattr(s, k)) for k, _ in StageStats._fields_}


class Lru(_Handle):
    """Host-only slot replacement policy (edge0_lru_*)."""

    def __init__(self, n_slots: int, n_layers: int, n_experts: int):
        self._handle = C.c_void_p()
        _check(lib.edge0_lru_create(C.byref(self._handle), n_slots, n_layers, n_experts),
               "edge0_lru_create")
        self._register()

    def request(self, layer: int, step: int, ids):
        """-> (slots, hit flags, evicted keys), each an int32 array."""
        ids = _i32(ids)
        n = ids.shape[0]
        slots, hit, ev = (np.zeros(n, np.int32) for _ in range(3))
        _check(lib.edge0_lru_request(self._handle, layer, step, _i32p(ids), n, _i32p(slots),
                                     _i32p(hit), _i32p(ev)), "edge0_lru_request")
        return slots, hit, ev

    def release(self, layer: int, step: int):
        _check(lib.edge0_lru_release(self._handle, layer, step), "edge0_lru_release")

    def stats(self) -> dict:
        s = StageStats()
        _check(lib.edge0_lru_stats(self._handle, C.byref(s)), "edge0_lru_stats")
        return _stats(s)

    def close(self):
        if self._handle:
            lib.edge0_lru_destroy(self._handle)
            self._handle = C.c_void_p()



EDGE0_FILE_DIRECT = 1


class FileStats(C.Structure):
    _fields_ = [("reads", C.c_int64), ("bytes", C.c_int64), ("read_ns", C.c_int64)]


def layer_file_write(path: str, shape: MoeShape, layer: int, bundle_ptrs):
    """Writes one layer's expert file from E host-readable bundle pointers."""
    arr = (C.c_void_p * len(bundle_ptrs))(*bundle_ptrs)
    _check(lib.edge0_layer_file_write(path.encode(), C.byref(shape), layer, arr),
           "edge0_layer_file_write")


class FileTier(_Handle):
    """Owner of an edge0_filetier handle: the open layer files, pinned staging
    buffers and I/O threads."""

    def __init__(self, shape: MoeShape, paths, n_buffers: int = 64, n_threads: int = 8,
                 direct: bool = True):
        self.shape = shape
        arr = (C.c_char_p * len(paths))(*[p.encode() for p in paths])
        self._handle = C.c_void_p()
        _check(lib.edge0_filetier_create(C.byref(self._handle), C.byref(shape), len(paths), arr,
                                         n_buffers, n_threads, EDGE0_FILE_DIRECT if direct else 0),
               "edge0_filetier_create")
        self._register()

    def stats(self) -> dict:
        s = FileStats()
        _check(lib.edge0_filetier_stats(self._handle, C.byref(s)), "edge0_filetier_stats")
        return {k: int(getattr(s, k)) for k, _ in FileStats._fields_}

    def close(self):
        if self._handle:
            lib.edge0_filetier_destroy(self._handle)
            self._handle = C.c_void_p()


class Stager(_Handle):
    """Owner of an edge0_stager handle: the LRU pool plus host-to-device
    staging, from pinned host bundles (host_ptrs) or from a FileTier."""

    def __init__(self, shape: MoeShape, pool: SlotPool, n_layers: int, host_ptrs, slot_table,
                 files: "FileTier | None" = None):
        self._keep = (host_ptrs, slot_table, files)
        self._handle = C.c_void_p()
        if files is not None:
            _check(lib.edge0_stager_create_files(C.byref(self._handle), C.byref(shape),
                                                 C.byref(pool), n_layers, files._handle,
                                                 _ptr(slot_table)), "edge0_stager_create_files")
        else:
            arr = (C.c_void_p * len(host_ptrs))(*host_ptrs)
            _check(lib.edge0_stager_create(C.byref(self._handle), C.byref(shape), C.byref(pool),
                                           n_layers, arr, _ptr(slot_table)), "edge0_stager_create")
        self._register()

    def stage(self, layer: int, step: int, ids, stream=None) -> np.ndarray:
        ids = _i32(ids)
        slots = np.zeros(ids.shape[0], np.int32)
        _check(lib.edge0_stage_experts(self._handle, layer, step, _i32p(ids), ids.shape[0],
                                       _i32p(slots), _stream(stream)), "edge0_stage_experts")
        return slots

    def wait(self, layer: int, step: int, stream=None):
        _check(lib.edge0_stager_wait(self._handle, layer, step, _stream(stream)),
               "edge0_stager_wait")

    def release(self, layer: int, step: int, stream=None):
        _check(lib.edge0_stager_release(self._handle, layer, step, _stream(stream)),
               "edge0_stager_release")

    def set_copy_mode(self, mode: int):
        """0: fill kernel (default); 1: DMA copies (hipMemcpyAsync)."""
        _check(lib.edge0_stager_set_copy_mode(self._handle, mode), "edge0_stager_set_copy_mode")

    def flush(self, stream=None):
        _check(lib.edge0_stager_flush(self._handle, _stream(stream)), "edge0_stager_flush")

    def stats(self) -> dict:
        s = StageStats()
        _check(lib.edge0_stager_stats(self._handle, C.byref(s)), "edge0_stager_stats")
        return _stats(s)

    def close(self):
        if self._handle:
            lib.edge0_stager_destroy(self._handle)
            self._handle = C.c_void_p()



def stack_step_staged(stack: "Stack", stager: Stager, h0, h_out, step: int, ids_dev, ids_host,
                      next_ids_host, ahead, copy_stream, stream=None):
    """One staged decode step (edge0_stack_step_staged).  ids_host and
    next_ids_host are int32 numpy arrays [n_layers][K] (next may be None);
    ahead is False/True (on demand / prediction arm over the given routing)
    or EDGE0_STAGE_LOOP (routing from the device, ids_* None)."""
    mode = EDGE0_STAGE_LOOP if ahead == EDGE0_STAGE_LOOP else (1 if ahead else 0)
    ids_host = None if ids_host is None else _i32(ids_host)
    nxt = None if next_ids_host is None else _i32(next_ids_host)
    plan = StagePlan(_ptr(ids_dev), None if ids_host is None else ids_host.ctypes.data,
                     None if nxt is None else nxt.ctypes.data, mode, _stream(copy_stream))
    _check(lib.edge0_stack_step_staged(stack._handle, stager._handle, C.byref(plan), _ptr(h0),
                                       _ptr(h_out), step, _stream(stream)),
           "edge0_stack_step_staged")


_hip = C.CDLL("libamdhip64.so")
_hip.hipMemcpy.restype = C.c_int
_hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]


def _wrap(ptr: int, shape, dtype) -> torch.Tensor:
    """Copy a device buffer owned by the library into a new torch tensor."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype, device="cuda")
    torch.cuda.synchronize()
    if _hip.hipMemcpy(out.data_ptr(), ptr, n * out.element_size(), 3) != 0:  # device to device
        raise RuntimeError("hipMemcpy failed")
    return out.view(*shape)
