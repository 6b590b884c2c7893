"""Plain fp64 CPU oracle for one decode step of an Edge0-style streaming MoE.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [Edge0]     "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
              with Trained Routing Prediction" (arXiv HTML).
  [Review]    jaehun.me review "Waking the MoE on SSD: Serving a 35B MoE at
              20 tok/s on a 24 GB Desktop with Edge0".
  [Cacheable] "Cacheable by Design?" (arXiv 2608.18261 full text).

Conventions.  Inputs arrive in their storage dtypes: bf16 as uint16 bit
patterns, fp16 as numpy float16, packed int4 as uint32 words.  Every such
value converts to fp64 exactly, and all arithmetic below is fp64 with numpy
library matrix-vector products as the only non-elementwise primitive.  Layer
outputs are returned unrounded; the stack rounds to bf16 exactly where the
method hands bf16 from one layer to the next.

Decisions taken on floating point: softmax-top-K ranks experts on the
logits rounded to fp32 (the precision the GPU ranks in), ties to the lower
index; sigmoid-group ranks groups and experts on fp32 scores built from the
sigmoid rounded once to fp32 (see sigmoid_group_topk).

Readings of points the pages leave open are stated where they are used and
listed with the design notes.  Every function here is pinned by CPU tests
(tests/test_oracle_pins.py; topk_gap, which decides the near-tie waivers, in
tests/test_tolerances.py).  Not a property of this code, and so not pinned:
the prediction quality of the heads (their weights are random).
"""
from __future__ import annotations

import math
from collections import Counter

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16_bits", "unpack_int4", "dequant", "lora_proj",
    "silu", "gelu_erf", "expert_ffn", "moe_layer", "router_logits",
    "softmax_topk", "softmax_at", "prerouter_feature", "prerouter_logits", "prerouter_commit",
    "rmsnorm", "stack_layer", "stack_step", "canonical_requests", "lru_replay",
    "grouped_layer", "topk_gap", "sigmoid_group_topk", "sigmoid_group_gaps", "NoSlotError",
    "lora_delta", "requantize_affine", "merge_requant", "layer_retention",
]


# --------------------------------------------------------------------------
# storage dtypes
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """fp64 -> bf16 bit pattern, one rounding to nearest (ties to even).

    bf16 keeps 8 significant bits: write v = m * 2^e with 0.5 <= |m| < 1 and
    round m * 2^8 to the nearest integer (np.rint rounds halves to even)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)      # exactly representable in bf16
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# int4 affine group quantisation   [Edge0] §2 "Quantization" (int4 affine,
# group 64); §3.1 "Executor paths" (weights, scales and biases per projection)
# --------------------------------------------------------------------------
def unpack_int4(words, n_in: int) -> np.ndarray:
    """Codes q[out][n_in] from u32 words[out][n_in/8]: input index i sits in
    word i//8 at bits 4*(i%8) (reading: low nibble holds the lowest index)."""
    w = np.asarray(words, dtype=np.uint32)
    assert w.shape[1] * 8 == n_in
    q = np.empty((w.shape[0], n_in), dtype=np.uint8)
    for j in range(8):
        q[:, j::8] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return q


def dequant(words, s_bits, b_bits, group: int) -> np.ndarray:
    """W[o][i] = s[o][i//g] * q[o][i] + b[o][i//g] (reading: additive bias,
    groups run along the input axis)."""
    s = bf16_to_f64(s_bits)
    b = bf16_to_f64(b_bits)
    n_in = s.shape[1] * group
    q = unpack_int4(words, n_in).astype(np.float64)
    return np.repeat(s, group, axis=1) * q + np.repeat(b, group, axis=1)


# --------------------------------------------------------------------------
# recovery LoRA   [Edge0] §3.3 (unmerged parallel delta y = W x + (a/r) B A x);
# Figure 1 (sum node)
# --------------------------------------------------------------------------
def lora_proj(W: np.ndarray, x: np.ndarray, A=None, B=None, scale: float = 0.0) -> np.ndarray:
    """Base product plus the unmerged delta: W x + scale * (B (A x)).
    A, B are bf16 bit arrays [r][in], [out][r]; None means no adapter."""
    base = W @ x
    if A is None:
        return base
    t = bf16_to_f64(A) @ x
    return base + scale * (bf16_to_f64(B) @ t)


# --------------------------------------------------------------------------
# activations
# --------------------------------------------------------------------------
def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z)   [Edge0] §3.1 "Math contract"."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu_erf(z):
    """Exact (erf) GELU: 0.5 z (1 + erf(z / sqrt 2))   [Edge0] §3.2 "Head"."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


# --------------------------------------------------------------------------
# expert FFN and the weighted combine   [Edge0] §3.1 "Math contract"
# (down(silu(gate(x)) * up(x)) over the routed experts)
# --------------------------------------------------------------------------
def expert_ffn(ex: dict, x: np.ndarray, group: int, lora: dict | None = None,
               scale: float = 0.0) -> np.ndarray:
    """One expert: G = gate(x), U = up(x), h = silu(G) * U, D = down(h); each
    projection carries its own unmerged LoRA delta when ``lora`` is given."""
    def proj(name, v):
        W = dequant(ex[name + "_q"], ex[name + "_s"], ex[name + "_b"], group)
        if lora is None:
            return lora_proj(W, v)
        return lora_proj(W, v, lora["a_" + name], lora["b_" + name], scale)

    G = proj("gate", x)
    U = proj("up", x)
    h = silu(G) * U
    return proj("down", h)


def moe_layer(experts, ids, w, x_bits, group: int, lora=None, scale: float = 0.0) -> np.ndarray:
    """y = sum_k w_k * FFN_{ids_k}(x), summed in the order the routing lists
    the ids; fp64, unrounded.  ``experts``/``lora`` map expert id -> arrays."""
    x = bf16_to_f64(x_bits)
    y = None
    for e, wk in zip(ids, w):
        e = int(e)
        D = expert_ffn(experts[e], x, group, None if lora is None else lora[e], scale)
        y = wk * D if y is None else y + wk * D
    return y


# --------------------------------------------------------------------------
# routing   [Edge0] §2 "MoE routing"; App. A "Softmax-topk"
# --------------------------------------------------------------------------
def router_logits(wr_bits, x_bits) -> np.ndarray:
    """Plain router: l = W_r x."""
    return bf16_to_f64(wr_bits) @ bf16_to_f64(x_bits)


def softmax_topk(logits, k: int):
    """g = softmax(l); ids = top-k(g, k); w = g[ids] / sum(g[ids]).

    Softmax is strictly increasing, so the top-k of g is the top-k of l; the
    ranking is taken on l rounded to fp32, in order of (value descending,
    index ascending).  Weights use the literal formula in fp64."""
    l = np.asarray(logits, dtype=np.float64)
    key = l.astype(np.float32)
    order = sorted(range(l.shape[0]), key=lambda e: (-float(key[e]), e))
    ids = np.array(order[:k], dtype=np.int32)
    g = np.exp(l - l.max())
    g = g / g.sum()
    w = g[ids] / g[ids].sum()
    return ids, w


def softmax_at(logits, ids) -> np.ndarray:
    """Weights of a routing whose ids are given rather than chosen:
    g = softmax(l) over all experts, w = g[ids] / sum(g[ids]) (the weight
    line of [Edge0] App. A "Softmax-topk", applied to the given set)."""
    l = np.asarray(logits, dtype=np.float64)
    g = np.exp(l - l.max())
    g = g / g.sum()
    ids = np.asarray(ids, dtype=np.int64)
    return g[ids] / g[ids].sum()


def topk_gap(logits, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest logit (inf when k = E)."""
    s = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    return float("inf") if k >= s.shape[0] else float(s[k - 1] - s[k])


def _sigmoid64(l: np.ndarray) -> np.ndarray:
    """sigmoid(l) = 1 / (1 + e^-l) in fp64 (e^-l overflowing gives 0)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-l))


def _sigmoid_group_scores(logits, n_groups: int, bias):
    """fp32 selection scores c = fp32(fp32(sigmoid(l)) + bias) and the fp32
    group scores (sum of each group's two largest c, largest first)."""
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[0]
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, dtype=np.float32)
    c = (_sigmoid64(l).astype(np.float32) + b).astype(np.float32)
    gs = E // n_groups
    gscore = np.empty(n_groups, np.float32)
    for i in range(n_groups):
        top = sorted((float(c[e]) for e in range(i * gs, (i + 1) * gs)), reverse=True)
        gscore[i] = np.float32(np.float32(top[0]) + np.float32(top[1]))
    return c, gscore


def sigmoid_group_topk(logits, k: int, n_groups: int, top_groups: int, scale: float,
                       bias=None):
    """Sigmoid-group routing, [Edge0] App. A "Sigmoid-group (K, G of n
    groups, scale s)" and §2 "MoE routing" (the DeepSeek-V3 family):

      sigma = sigmoid(l)
      c     = sigma + bias          (selection score; bias = 0 when absent)
      group i = experts [i E/n, (i+1) E/n); its score = the sum of its two
              largest c; the top_groups groups by score survive, the others
              are masked out
      ids   = the k largest c among the surviving experts
      w     = scale * sigma[ids] / (sum sigma[ids] + 1e-20)

    Readings: the appendix says selection uses a biased score without
    printing the bias, so the bias is a per-expert vector added to sigma
    for the group scores and the top-k only, while the weights use the raw
    sigma; groups are contiguous runs of E/n experts.  Decisions are taken
    in fp32 (the precision the GPU decides in): sigma rounded once to fp32,
    c and the group sums fp32 additions; groups and experts rank by (score
    descending, index ascending).  ids are listed in that rank order.
    Weights are fp64 on the fp64 sigma."""
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[0]
    if n_groups < 1 or E % n_groups or E // n_groups < 2 or not 1 <= top_groups <= n_groups:
        raise ValueError("sigmoid-group routing needs E % n == 0, E / n >= 2, 1 <= G <= n")
    gs = E // n_groups
    if not 1 <= k <= top_groups * gs:
        raise ValueError("k must not exceed the experts of the surviving groups")
    c, gscore = _sigmoid_group_scores(l, n_groups, bias)
    keep = sorted(range(n_groups), key=lambda i: (-float(gscore[i]), i))[:top_groups]
    alive = [e for i in keep for e in range(i * gs, (i + 1) * gs)]
    ids = np.array(sorted(alive, key=lambda e: (-float(c[e]), e))[:k], dtype=np.int32)
    sig = _sigmoid64(l)
    w = scale * sig[ids] / (sig[ids].sum() + 1e-20)
    return ids, w


def sigmoid_group_gaps(logits, k: int, n_groups: int, top_groups: int, bias=None):
    """The two margins a sigmoid-group decision rests on: between the
    top_groups-th and next group score (inf when every group survives), and
    between the k-th and (k+1)-th selection score among the surviving
    experts (inf when all of them are taken).  A difference of a few fp32
    ulps in sigma can flip a decision whose margin is that small."""
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[0]
    gs = E // n_groups
    c, gscore = _sigmoid_group_scores(l, n_groups, bias)
    gsorted = sorted((float(v) for v in gscore), reverse=True)
    ggap = float("inf") if top_groups >= n_groups else gsorted[top_groups - 1] - gsorted[top_groups]
    keep = sorted(range(n_groups), key=lambda i: (-float(gscore[i]), i))[:top_groups]
    alive = sorted((float(c[e]) for i in keep for e in range(i * gs, (i + 1) * gs)), reverse=True)
    egap = float("inf") if k >= len(alive) else alive[k - 1] - alive[k]
    return ggap, egap


# --------------------------------------------------------------------------
# prerouter head   [Edge0] §3.2 "Head", "Prediction-as-routing",
# "Feature drift"; [Review] toy example (8 + 2*4 = 16-dim feature)
# --------------------------------------------------------------------------
def prerouter_feature(x_bits, ids_now, ids_prev, n_experts: int) -> np.ndarray:
    """f = [x ; onehot(ids_now) ; onehot(ids_prev)], dim d + 2E.  One-hots are
    binary multi-hots with one 1 per routed expert; ids_prev None = zeros."""
    x = bf16_to_f64(x_bits)
    now = np.zeros(n_experts)
    now[np.asarray(ids_now, dtype=np.int64)] = 1.0
    prev = np.zeros(n_experts)
    if ids_prev is not None:
        prev[np.asarray(ids_prev, dtype=np.int64)] = 1.0
    return np.concatenate([x, now, prev])


def prerouter_logits(head: dict, x_bits, ids_now, ids_prev, n_experts: int) -> np.ndarray:
    """logits = fc2(gelu(fc1(f))) + l(x), with fc1 = [w1x | w1oh^T] acting on
    the dense feature f, fc2 = w2, residual l = wl (reads the hidden part
    only, no bias).  Missing biases (None) are zero."""
    f = prerouter_feature(x_bits, ids_now, ids_prev, n_experts)
    W1 = np.concatenate([head["w1x"].astype(np.float64),
                         head["w1oh"].astype(np.float64).T], axis=1)
    z1 = W1 @ f
    if head.get("b1") is not None:
        z1 = z1 + head["b1"].astype(np.float64)
    a = gelu_erf(z1)
    logits = head["w2"].astype(np.float64) @ a
    if head.get("b2") is not None:
        logits = logits + head["b2"].astype(np.float64)
    if head.get("wl") is not None:
        logits = logits + head["wl"].astype(np.float64) @ bf16_to_f64(x_bits)
    return logits


def prerouter_commit(head: dict, x_bits, ids_now, ids_prev, n_experts: int, k: int):
    """The prediction for layer N+1 at token t+1 made by the head owned by
    layer N at token t, committed as that layer's routing through the same
    softmax-top-k (weights from the head's logits).  Returns (ids, w, logits)."""
    logits = prerouter_logits(head, x_bits, ids_now, ids_prev, n_experts)
    ids, w = softmax_topk(logits, k)
    return ids, w, logits


# --------------------------------------------------------------------------
# synthetic stack   (random-init layers with RMSNorm between them)
# --------------------------------------------------------------------------
def rmsnorm(h, eps: float = 1e-6) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps), unit gain (reading: eps 1e-6, gamma 1)."""
    h = np.asarray(h, dtype=np.float64)
    return h / math.sqrt(float(np.mean(h * h)) + eps)


def stack_layer(layer, h_bits, shape, *, routing=None, ids_prev=None, run_head=False,
                eps: float = 1e-6) -> dict:
    """One pre-norm residual block without attention:
        x = bf16(RMSNorm(h)); routing = given (committed) or softmax-top-k of
        the plain router; y = MoE(x); h' = bf16(h + bf16(y)).
    When ``run_head`` the layer's head predicts the next layer's routing at
    the next token from x, this token's executed ids and the previous
    token's ids of this layer (feature drift: the executed routing).
    ``layer`` provides: expert(e) -> arrays, lora(e) -> arrays or None,
    router -> bf16 bits, head -> dict."""
    h = bf16_to_f64(h_bits)
    x_bits = f64_to_bf16_bits(rmsnorm(h, eps))
    logits = None
    if routing is None:
        logits = router_logits(layer.router, x_bits)
        ids, w = softmax_topk(logits, shape.top_k)
    else:
        ids, w = routing
    scale = shape.lora_alpha / shape.lora_rank if shape.lora_rank else 0.0
    experts = {int(e): layer.expert(int(e)) for e in ids}
    lora = None
    if shape.lora_rank:
        lora = {int(e): layer.lora(int(e)) for e in ids}
    y = moe_layer(experts, ids, w, x_bits, shape.group, lora, scale)
    y_bits = f64_to_bf16_bits(y)
    h_next = f64_to_bf16_bits(h + bf16_to_f64(y_bits))
    pred = None
    if run_head:
        pred = prerouter_commit(layer.head, x_bits, ids, ids_prev, shape.n_experts, shape.top_k)
    return {"x": x_bits, "ids": np.asarray(ids, np.int32), "w": np.asarray(w),
            "router_logits": logits, "y": y, "y_bits": y_bits, "h_next": h_next, "pred": pred}


def stack_step(layers, h0_bits, t: int, committed: dict, prev_ids: dict, shape,
               owners=range(6, 38), consumers=range(7, 39), eps: float = 1e-6):
    """One decode step through the stack (reading of the owner/consumer
    ranges: heads owned by 6..37 run, layers 7..38 route by the prediction
    committed at the previous token, the rest - and every layer at t = 0 -
    by the plain router).  ``committed`` maps layer -> (ids, w) predicted at
    t-1; ``prev_ids`` maps layer -> ids executed at t-1.  Returns
    (h_out_bits, per-layer results, committed for t+1, executed ids)."""
    h = h0_bits
    out, new_committed, executed = [], {}, {}
    for L, layer in enumerate(layers):
        routing = committed[L] if (L in consumers and t > 0) else None
        r = stack_layer(layer, h, shape, routing=routing, ids_prev=prev_ids.get(L),
                        run_head=(L in owners), eps=eps)
        if r["pred"] is not None:
            new_committed[L + 1] = (r["pred"][0], r["pred"][1])
        executed[L] = r["ids"]
        out.append(r)
        h = r["h_next"]
    return h, out, new_committed, executed


# --------------------------------------------------------------------------
# bounded slot pool with LRU replacement   [Edge0] Figure 1 (bounded
# streaming pool: LRU, staged fixed-slot double buffer), §3.1 "Executor
# paths" (slot table), Table 1 caption (shared LRU of expert bundles);
# [Cacheable] App. E (LRU cache replay)
# --------------------------------------------------------------------------
class NoSlotError(RuntimeError):
    pass


def canonical_requests(n_steps: int, n_layers: int, owners=range(6, 38),
                       consumers=range(7, 39), heads_at_end: bool = False):
    """Request/consume events in the canonical host order, per step t and
    layer L: a layer that does not consume a prediction (or any layer at
    t = 0) requests its own set right before it computes; every layer
    consumes its set when it computes; once the head of owner layer L has
    run, the set predicted for (L+1, t+1) is requested.  A head runs right
    after its layer, or - with ``heads_at_end``, the heads of a step flushed
    as one batch after its last layer ([Edge0] §3.2 "Head": one flush per
    step) - after the step's last layer, in owner order."""
    ev = []
    for t in range(n_steps):
        for L in range(n_layers):
            if not (L in consumers and t > 0):
                ev.append(("req", L, t))
            ev.append(("use", L, t))
            if L in owners and not heads_at_end:
                ev.append(("req", L + 1, t + 1))
        if heads_at_end:
            ev.extend(("req", L + 1, t + 1) for L in owners)
    return ev


def lru_replay(events, ids_of, n_slots: int):
    """Replay requests against one pool of ``n_slots`` slots shared by all
    layers.  ``ids_of(L, t)`` gives the set of a request.

    A request pins every (L, id) of its set until the matching "use".  Its
    ids are then taken in order: a resident id is a hit; a missing id takes
    the lowest free slot, else evicts the unpinned slot with the oldest
    stamp.  Every touched id gets a new stamp from one global counter, so
    stamps are unique and eviction never ties.  Returns a list of per-request
    records {"L","t","ids","slots","hit","evicted"} and totals."""
    owner = [None] * n_slots
    stamp = [0] * n_slots
    slot_of = {}
    pinned = Counter()
    pending = {}
    clock = 0
    records = []
    hits = misses = 0
    for kind, L, t in events:
        if kind == "use":
            for e in pending.pop((L, t)):
                pinned[(L, e)] -= 1
            continue
        ids = [int(e) for e in ids_of(L, t)]
        pending[(L, t)] = ids
        for e in ids:
            pinned[(L, e)] += 1
        slots, hit, evicted = [], [], []
        for e in ids:
            clock += 1
            key = (L, e)
            if key in slot_of:
                s = slot_of[key]
                hit.append(True)
                hits += 1
            else:
                free = [i for i in range(n_slots) if owner[i] is None]
                if free:
                    s = free[0]
                    evicted.append(None)
                else:
                    cand = [i for i in range(n_slots) if pinned[owner[i]] == 0]
                    if not cand:
                        raise NoSlotError(f"every slot is pinned at request ({L}, {t})")
                    s = min(cand, key=lambda i: stamp[i])
                    evicted.append(owner[s])
                    del slot_of[owner[s]]
                owner[s] = key
                slot_of[key] = s
                hit.append(False)
                misses += 1
            stamp[s] = clock
            slots.append(s)
        records.append({"L": L, "t": t, "ids": ids, "slots": slots, "hit": hit,
                        "evicted": evicted})
    return records, {"hits": hits, "misses": misses, "touches": hits + misses}


# --------------------------------------------------------------------------
# several tokens per step: defined token by token (grouping is scheduling)
# --------------------------------------------------------------------------
def grouped_layer(experts, ids, w, x_bits, group: int, lora=None, scale: float = 0.0):
    """y_j = sum_k w[j,k] FFN_{ids[j,k]}(x_j) for every token j."""
    return np.stack([moe_layer(experts, ids[j], w[j], x_bits[j], group, lora, scale)
                     for j in range(ids.shape[0])])


# --------------------------------------------------------------------------
# merging the LoRA into the int4 weights   [Edge0] §3.3 "Recovery LoRA:
# Unmerged by Design" and its footnote 2 (weight-level retention)
# --------------------------------------------------------------------------
def lora_delta(A_bits, B_bits, scale: float) -> np.ndarray:
    """delta = scale * B A  ([out][in], fp64), the LoRA's change of the weight."""
    return scale * (bf16_to_f64(B_bits) @ bf16_to_f64(A_bits))


def requantize_affine(W: np.ndarray, group: int):
    """int4 affine quantisation of W [out][in] per group of `group` inputs
    (reading: the plain min/max quantiser of the format, [Edge0] §2
    "Quantization"): s = (max - min) / 15 and b = min, each rounded to bf16;
    q = round((w - b) / s) to nearest (ties to even), clipped to 0..15; a
    group whose s rounds to 0 keeps q = 0.  Returns (q, s bits, b bits)."""
    W = np.asarray(W, dtype=np.float64)
    out_dim, in_dim = W.shape
    Wg = W.reshape(out_dim, in_dim // group, group)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    s_bits = f64_to_bf16_bits((hi - lo) / 15.0)
    b_bits = f64_to_bf16_bits(lo)
    s = bf16_to_f64(s_bits)[:, :, None]
    b = bf16_to_f64(b_bits)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((Wg - b) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, 15).astype(np.int64).reshape(out_dim, in_dim)
    return q, s_bits, b_bits


def merge_requant(words, s_bits, b_bits, A_bits, B_bits, scale: float, group: int):
    """The merge the pages reject: W' = dequant(W) + delta, requantised to
    int4.  Returns the requantised (q, s, b), the change that survived,
    actual = dequant(W'') - dequant(W), and the weight-level retention
    sum(actual * delta) / sum(delta^2) ([Edge0] §3.3, footnote 2)."""
    W = dequant(words, s_bits, b_bits, group)
    delta = lora_delta(A_bits, B_bits, scale)
    q, s2, b2 = requantize_affine(W + delta, group)
    g = group
    Wr = (bf16_to_f64(s2).repeat(g, axis=1) * q + bf16_to_f64(b2).repeat(g, axis=1))
    actual = Wr - W
    den = float(np.sum(delta * delta))
    return (q, s2, b2), actual, (float(np.sum(actual * delta)) / den if den > 0 else float("nan"))


def layer_retention(y_unmerged, y_merged, y_base) -> float:
    """Output-level retention 1 - |U - M| / |U - B| ([Edge0] §3.3, footnote
    2, taken on a layer's output here rather than on the logits): U with
    the unmerged LoRA, M on the merged and requantised weights, B on the
    base weights alone."""
    U, M, B = (np.asarray(v, dtype=np.float64) for v in (y_unmerged, y_merged, y_base))
    return 1.0 - float(np.linalg.norm(U - M) / np.linalg.norm(U - B))
