"""Shared helpers for the GPU parity tests: a seeded layer uploaded to the
device, and the comparison rules (rel-L2 on outputs, bit-exact ids with the
near-tie waiver, rel 1e-5 on routing weights)."""
from __future__ import annotations

import numpy as np

import oracle as O
from synth import gen as G

REL_L2_MAX = 2e-3      # layer outputs, bf16 I/O with fp32 accumulation
W_REL_MAX = 1e-5       # routing weights
TIE_GAP = 1e-4         # ids are compared bit-exactly unless a gap is below this


# Relative error bound of an fp32 RMSNorm output before its bf16 rounding,
# x = h * (1 / sqrt(sum(h^2) / d + eps)) with bf16 h (so each h^2 is exact in
# fp32).  A sum of positive terms carries at most (rounding levels on its
# longest path) * u relative error, u = 2^-24; the kernels sum at most 8
# terms per thread and then reduce over at most 256 threads in a tree: at
# most 17 levels, 17u.  The square root halves that (8.5u); adding eps, the
# root, the reciprocal and the final product add at most 4u: 12.5u = 7.5e-7.
# 1e-6 (16.8u) covers it; an eps off by 9e-6 (1e-5 in place of 1e-6) shifts
# x by 4.5e-6 relative and is caught (tests/test_tolerances.py).
RMSNORM_REL = 1e-6


def check_bf16_rounding(got_bits, exact, rel=RMSNORM_REL):
    """A bf16 vector computed in fp32 against its exact fp64 value: every
    element is the round-to-nearest-even of the exact value, except where the
    exact value lies within `rel` (the fp32 error bound of the computation,
    RMSNORM_REL) of the midpoint between two bf16 neighbours; there either
    neighbour is correct.  Returns the number of such near-midpoint elements
    that rounded the other way."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    exact = np.asarray(exact, dtype=np.float64)
    want = O.f64_to_bf16_bits(exact)
    diff = np.nonzero(got_bits != want)[0]
    if diff.size == 0:
        return 0
    g = O.bf16_to_f64(got_bits[diff])
    w = O.bf16_to_f64(want[diff])
    e = exact[diff]
    lo, hi = np.minimum(g, w), np.maximum(g, w)
    # the two values must be adjacent bf16 numbers bracketing the exact value
    step = hi - lo
    bits_lo = O.f64_to_bf16_bits(lo).astype(np.int32)
    bits_hi = O.f64_to_bf16_bits(hi).astype(np.int32)
    adjacent = (np.abs(bits_hi - bits_lo) == 1) | ((lo < 0) & (hi > 0))
    assert adjacent.all(), (diff[~adjacent], g[~adjacent], w[~adjacent])
    assert ((e >= lo) & (e <= hi)).all(), diff
    mid = (lo + hi) / 2
    near = np.abs(e - mid) <= rel * np.abs(e) + 1e-300
    assert near.all(), (diff[~near], e[~near], mid[~near], step[~near])
    return int(diff.size)


# Layer outputs, element by element: within one bf16 step of the exact value
# (a correctly rounded result is within half a step; the kernel's fp32 value
# may sit on the other side of a rounding midpoint), plus an absolute floor
# for the fp32 computation's own error, Y_ABS_RMS * rms(y): the SwiGLU output
# enters the down projection as a bf16 hi/lo pair (16 significant bits,
# 2^-17 = 7.6e-6 relative), which with the fp32 sums stays within a few
# times that of the row's scale.
Y_ABS_RMS = 3e-5
# rel-L2 allowed beyond the bf16 rounding of the exact output itself: an
# output's rounding alone costs 1.6e-3 on average, and at d = 256 its spread
# between tokens reaches the flat 2e-3 bar.
Y_REL_OVER_ROUNDING = 2e-4


def check_layer_output(got_bits, exact):
    """One layer output (bf16 bits) against the exact fp64 value: rel-L2 at
    most REL_L2_MAX or at most Y_REL_OVER_ROUNDING above the rounding of the
    exact value itself, and every element within one bf16 step plus
    Y_ABS_RMS * rms.  Returns (rel-L2, worst element error in steps)."""
    g = O.bf16_to_f64(np.asarray(got_bits, dtype=np.uint16))
    e = np.asarray(exact, dtype=np.float64)
    rel = rel_l2(g, e)
    r_round = rel_l2(O.bf16_to_f64(O.f64_to_bf16_bits(e)), e)
    assert rel <= REL_L2_MAX or rel <= r_round + Y_REL_OVER_ROUNDING, (rel, r_round)
    mag = np.maximum(np.abs(g), np.abs(e))
    step = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-300))) - 7)
    err = np.abs(g - e)
    rms = float(np.sqrt(np.mean(e * e)))
    bad = err > step + Y_ABS_RMS * rms
    assert not bad.any(), (np.nonzero(bad)[0][:8], err[bad][:8], step[bad][:8], rms)
    return rel, float(np.max(err / (step + Y_ABS_RMS * rms)))


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def check_routing(gpu_ids, gpu_w, logits, k):
    """Compare a GPU top-K against the oracle's on the oracle's logits.
    Returns "exact" or "waived" (near tie at the K-th place); raises on a
    mismatch.  Within the set, order may differ only between logits closer
    than TIE_GAP; weights are compared per id."""
    gpu_ids = np.asarray(gpu_ids)
    ids, w = O.softmax_topk(logits, k)
    if O.topk_gap(logits, k) < TIE_GAP:
        return "waived"
    assert sorted(gpu_ids.tolist()) == sorted(ids.tolist()), (gpu_ids, ids)
    for a, b in zip(gpu_ids, ids):
        if a != b:
            assert abs(logits[a] - logits[b]) < TIE_GAP, (gpu_ids, ids)
    want = dict(zip(ids.tolist(), w.tolist()))
    for e, wv in zip(gpu_ids.tolist(), np.asarray(gpu_w, dtype=np.float64).tolist()):
        assert abs(wv - want[e]) <= W_REL_MAX * abs(want[e]), (e, wv, want[e])
    return "exact"


class DeviceLayer:
    """One seeded MoE layer (all E experts in slots 0..E-1 of a pool, or
    permuted), its router and head, on the GPU."""

    def __init__(self, S, seed=0, layer=0, slot_perm=None, lora=True, free_bias=False,
                 scales=G.DEFAULT_SCALES):
        import torch
        from int4_expert_streaming_amd import edge0 as E
        from int4_expert_streaming_amd.weights import SlotPoolBuffer, to_device, head_to_device
        self.S = S
        self.E = E
        self.sh = E.make_shape(S)
        if not lora:
            self.sh.lora_rank = 0
        self.experts = {e: G.expert_tensors(S, seed, layer, e, free_bias=free_bias, scales=scales)
                        for e in range(S.n_experts)}
        self.loras = ({e: G.lora_tensors(S, seed, layer, e) for e in range(S.n_experts)}
                      if lora else None)
        perm = np.arange(S.n_experts) if slot_perm is None else np.asarray(slot_perm)
        self.pool = SlotPoolBuffer(self.sh, S.n_experts)
        for e in range(S.n_experts):
            self.pool.load(int(perm[e]), self.experts[e], None if not lora else self.loras[e])
        self.table = torch.tensor(perm, dtype=torch.int32, device="cuda")
        self.wr = G.router_weight(S, seed, layer)
        self.wr_d = to_device(self.wr)
        self.head = G.head_tensors(S, seed, layer)
        self.head_d = head_to_device(self.head)
        self.ws = E.new_workspace(self.sh)
        self.scale = S.lora_alpha / S.lora_rank if lora else 0.0

    def new_routing(self):
        import torch
        K = self.S.top_k
        return (torch.zeros(K, dtype=torch.int32, device="cuda"),
                torch.zeros(K, dtype=torch.float32, device="cuda"))

    def oracle_y(self, ids, w, x_bits):
        return O.moe_layer(self.experts, np.asarray(ids), np.asarray(w, dtype=np.float64), x_bits,
                           self.S.group, self.loras, self.scale)
