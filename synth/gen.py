"""Seeded synthetic inputs for the streaming-MoE decode path.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``SeedSequence(seed, spawn_key=(kind, layer, expert, tensor))`` so any single
tensor can be regenerated alone, in any order.  Values are drawn in float32
and rounded to the storage dtype with round-to-nearest-even; both the oracle
and the HIP path receive the rounded bit patterns.

Distributions (the pages give the shapes, the configs give the ranges):
  * int4 codes q ~ U{0..15}; a uniformly random u32 word is eight independent
    uniform nibbles, so packed weights are drawn as random words directly.
  * group scale s ~ U[0.005, 0.02] (bf16); group bias b = -8*s (exact in bf16),
    so dequantised weights s*q+b are centred on zero.  Opt-in variants for
    the tests: a bias drawn independently of the scale, b ~ U[-0.16, 0.04]
    (bf16), so a path that ignored b or derived it from s would show; and
    another scale range (e.g. much smaller scales).
  * LoRA A ~ N(0, 0.02^2), B ~ N(0, 0.01^2) (bf16).
  * router W_r ~ N(0, 1/d) (bf16) so that a unit-RMS hidden state gives
    logits of roughly unit variance.
  * prerouter head (fp16): fc1 ~ N(0, 1/(d+2E)), fc2 ~ N(0, 1/H),
    biases ~ N(0, 0.02^2), residual ~ N(0, 1/d).
  * hidden states ~ N(0, 1) (bf16).
  * routing traces: Zipf(1.1) popularity over a per-layer random permutation
    of the experts, with each expert of the previous token's set kept with a
    fixed probability (adjacent-token overlap control).

Nothing here dequantises, multiplies, routes or normalises: this module is
input preparation only.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "MoEShape", "TINY", "QWEN3_MOE", "rng_for", "to_bf16_bits", "to_fp16",
    "pack_int4", "expert_tensors", "lora_tensors", "head_tensors",
    "router_weight", "hidden", "stack_hidden", "zipf_probs",
    "zipf_trace", "grouped_routing", "EXPERT_KEYS", "LORA_KEYS", "HEAD_KEYS", "StackGen",
    "DEFAULT_SCALES", "FREE_BIAS_RANGE", "scale_pow2",
]


@dataclass(frozen=True)
class MoEShape:
    """One MoE layer's sizes (the spec a model is described by)."""
    d_model: int
    n_experts: int
    d_inter: int
    top_k: int
    group: int
    lora_rank: int
    lora_alpha: float
    head_hidden: int

    def with_k(self, k: int) -> "MoEShape":
        return MoEShape(self.d_model, self.n_experts, self.d_inter, k, self.group,
                        self.lora_rank, self.lora_alpha, self.head_hidden)


# Single tiny layer: hidden 256, 16 experts, inter 128, top-4, group 32,
# LoRA r=8 alpha=16, head 256+2*16 -> 64 -> 16.
TINY = MoEShape(256, 16, 128, 4, 32, 8, 16.0, 64)
# Qwen3-MoE-shaped layer: hidden 2048, 128 experts, inter 768, top-4 (or 8),
# group 64, LoRA r=16 alpha=32, head 2048+2*128 -> 512 -> 128.
QWEN3_MOE = MoEShape(2048, 128, 768, 4, 64, 16, 32.0, 512)

# stream kinds
_K_EXPERT, _K_LORA, _K_HEAD, _K_ROUTER, _K_HIDDEN, _K_TRACE, _K_GROUPED = 1, 2, 3, 4, 5, 6, 7

EXPERT_KEYS = ("gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b",
               "down_q", "down_s", "down_b")
LORA_KEYS = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")
HEAD_KEYS = ("w1x", "w1oh", "b1", "w2", "b2", "wl")


def rng_for(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def to_fp16(a) -> np.ndarray:
    """float32 -> fp16 (numpy's conversion rounds to nearest even)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack codes q[out][in] (0..15) as u32 words[out][in/8]; element i of a row
    sits in word i/8 at bits 4*(i%8) (lowest input index in the low nibble)."""
    q = np.asarray(q)
    out, n_in = q.shape
    assert n_in % 8 == 0 and q.min() >= 0 and q.max() <= 15
    q = q.astype(np.uint32).reshape(out, n_in // 8, 8)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    return np.bitwise_or.reduce(q << shifts, axis=-1).astype(np.uint32)


DEFAULT_SCALES = (0.005, 0.02)
FREE_BIAS_RANGE = (-0.16, 0.04)


def _scales_biases(rng, rows, groups, scales=DEFAULT_SCALES, bias_rng=None):
    s = to_bf16_bits(rng.uniform(scales[0], scales[1], size=(rows, groups)).astype(np.float32))
    if bias_rng is not None:              # independent of s
        b = to_bf16_bits(bias_rng.uniform(*FREE_BIAS_RANGE, size=(rows, groups)).astype(np.float32))
        return s, b
    s_f = (s.astype(np.uint32) << 16).view(np.float32)
    b = to_bf16_bits(-8.0 * s_f)            # exact: a power-of-two multiple of a bf16 value
    return s, b


def expert_tensors(shape: MoEShape, seed: int, layer: int, expert: int, *,
                   free_bias: bool = False, scales=DEFAULT_SCALES) -> dict:
    """The nine arrays of one expert bundle (gate, up, down x (q, s, b)).

    q: u32 [out][in/8]; s, b: bf16 bits [out][in/g].  gate/up are [I x d],
    down is [d x I].  free_bias: b drawn from its own stream, independent of
    s; scales: the range of s."""
    d, I, g = shape.d_model, shape.d_inter, shape.group
    out = {}
    for t, (name, rows, cols) in enumerate((("gate", I, d), ("up", I, d), ("down", d, I))):
        rng = rng_for(seed, _K_EXPERT, layer, expert, t)
        brng = rng_for(seed, _K_EXPERT, layer, expert, t, 1) if free_bias else None
        out[name + "_q"] = rng.integers(0, 2**32, size=(rows, cols // 8), dtype=np.uint32)
        out[name + "_s"], out[name + "_b"] = _scales_biases(rng, rows, cols // g, scales, brng)
    return out


def lora_tensors(shape: MoEShape, seed: int, layer: int, expert: int) -> dict:
    """Per-expert recovery-LoRA pair per projection (bf16 bits):
    a_gate [r][d], b_gate [I][r], a_up [r][d], b_up [I][r], a_down [r][I], b_down [d][r]."""
    d, I, r = shape.d_model, shape.d_inter, shape.lora_rank
    dims = {"gate": (d, I), "up": (d, I), "down": (I, d)}
    out = {}
    for t, proj in enumerate(("gate", "up", "down")):
        n_in, n_out = dims[proj]
        rng = rng_for(seed, _K_LORA, layer, expert, t)
        out["a_" + proj] = to_bf16_bits(rng.normal(0.0, 0.02, size=(r, n_in)).astype(np.float32))
        out["b_" + proj] = to_bf16_bits(rng.normal(0.0, 0.01, size=(n_out, r)).astype(np.float32))
    return out


def head_tensors(shape: MoEShape, seed: int, layer: int) -> dict:
    """Prerouter head owned by ``layer`` (fp16):
    w1x [H][d] (fc1, hidden-state columns), w1oh [2E][H] (fc1 one-hot columns,
    stored transposed: row e < E is expert e of this token's routing, row E+e
    is expert e of the previous token's), b1 [H], w2 [E][H], b2 [E],
    wl [E][d] (linear residual, no bias)."""
    d, E, H = shape.d_model, shape.n_experts, shape.head_hidden
    rng = rng_for(seed, _K_HEAD, layer)
    fan1 = 1.0 / np.sqrt(d + 2 * E)
    return {
        "w1x": to_fp16(rng.normal(0.0, fan1, size=(H, d))),
        "w1oh": to_fp16(rng.normal(0.0, fan1, size=(2 * E, H))),
        "b1": to_fp16(rng.normal(0.0, 0.02, size=(H,))),
        "w2": to_fp16(rng.normal(0.0, 1.0 / np.sqrt(H), size=(E, H))),
        "b2": to_fp16(rng.normal(0.0, 0.02, size=(E,))),
        "wl": to_fp16(rng.normal(0.0, 1.0 / np.sqrt(d), size=(E, d))),
    }


def router_weight(shape: MoEShape, seed: int, layer: int) -> np.ndarray:
    """Plain router matrix W_r [E][d] (bf16 bits)."""
    rng = rng_for(seed, _K_ROUTER, layer)
    return to_bf16_bits(rng.normal(0.0, 1.0 / np.sqrt(shape.d_model),
                                   size=(shape.n_experts, shape.d_model)).astype(np.float32))


def hidden(shape: MoEShape, seed: int, index: int = 0, n: int | None = None) -> np.ndarray:
    """Hidden vector(s) x ~ N(0,1) as bf16 bits: [d] or [n][d]."""
    rng = rng_for(seed, _K_HIDDEN, index)
    size = (shape.d_model,) if n is None else (n, shape.d_model)
    return to_bf16_bits(rng.normal(0.0, 1.0, size=size).astype(np.float32))


def scale_pow2(bits, k: int) -> np.ndarray:
    """bf16 bit patterns times 2^k (exact for results inside the normal
    range: only the exponent changes)."""
    f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return to_bf16_bits(np.ldexp(f, k).astype(np.float32))


def stack_hidden(shape: MoEShape, seed: int, step: int) -> np.ndarray:
    """Fresh per-step stack input h0_t ~ N(0,1) (bf16 bits) for decode step t."""
    return hidden(shape, seed, 1_000_000 + step)


def zipf_probs(n: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def _draw_distinct(rng, probs, k, exclude):
    """k distinct indices drawn without replacement with probability ~ probs,
    skipping ``exclude``; returned in draw order."""
    p = probs.copy()
    p[list(exclude)] = 0.0
    out = []
    for _ in range(k):
        c = rng.choice(len(p), p=p / p.sum())
        out.append(int(c))
        p[c] = 0.0
    return out


def zipf_trace(n_experts: int, k: int, n_layers: int, n_steps: int, seed: int,
               keep_p: float, s: float = 1.1) -> np.ndarray:
    """Routing trace ids[step][layer][k] (int32).

    Per layer a seeded permutation maps popularity rank to expert id, with
    P(rank r) ~ r^-s.  At step 0 the set is k distinct Zipf draws.  At step
    t > 0 each id of the previous set is kept with probability keep_p (kept ids
    first, in their previous order), and the rest are fresh distinct Zipf draws
    that avoid the kept ids."""
    ranks = zipf_probs(n_experts, s)
    ids = np.empty((n_steps, n_layers, k), dtype=np.int32)
    for layer in range(n_layers):
        rng = rng_for(seed, _K_TRACE, layer)
        perm = rng.permutation(n_experts)
        probs = np.empty(n_experts)
        probs[perm] = ranks                 # expert perm[r] has popularity rank r
        prev = None
        for t in range(n_steps):
            if prev is None:
                cur = _draw_distinct(rng, probs, k, ())
            else:
                kept = [e for e in prev if rng.random() < keep_p]
                cur = kept + _draw_distinct(rng, probs, k - len(kept), kept)
            ids[t, layer] = cur
            prev = cur
    return ids


def grouped_routing(n_experts: int, k: int, n_tokens: int, seed: int, layer: int = 0,
                    s: float = 1.1):
    """Multi-token routing: each token draws k distinct experts ~ Zipf(s) over a
    per-layer permutation; weights are positive random numbers scaled to sum 1.
    Returns ids int32 [T][k], w float32 [T][k]."""
    ranks = zipf_probs(n_experts, s)
    rng = rng_for(seed, _K_GROUPED, layer)
    perm = rng.permutation(n_experts)
    probs = np.empty(n_experts)
    probs[perm] = ranks
    ids = np.empty((n_tokens, k), dtype=np.int32)
    w = np.empty((n_tokens, k), dtype=np.float32)
    for j in range(n_tokens):
        ids[j] = _draw_distinct(rng, probs, k, ())
        u = rng.uniform(0.1, 1.0, size=k)
        w[j] = (u / u.sum()).astype(np.float32)
    return ids, w


class StackGen:
    """Per-layer generator callables of a seeded synthetic stack."""

    def __init__(self, shape: MoEShape, seed: int = 0, free_bias: bool = False):
        self.S, self.seed, self.free_bias = shape, seed, free_bias

    def expert(self, L, e):
        return expert_tensors(self.S, self.seed, L, e, free_bias=self.free_bias)

    def lora(self, L, e):
        return lora_tensors(self.S, self.seed, L, e)

    def router(self, L):
        return router_weight(self.S, self.seed, L)

    def head(self, L):
        return head_tensors(self.S, self.seed, L)
