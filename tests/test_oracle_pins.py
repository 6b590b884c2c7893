"""Pins of the CPU oracle to things other than itself: values the pages print,
hand-worked examples, closed forms, library routines and brute force.

Each test names what it pins.  All run on the CPU."""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
from synth import gen as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def bf(v):
    """float values (exactly representable in bf16) -> bf16 bits."""
    a = np.asarray(v, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), a), "not bf16-exact"
    return bits


# ---------------------------------------------------------------- storage
def test_unpack_hand_words():
    """Pins nibble order: hand-packed words decode to the listed codes."""
    for row in _lines("int4_words.txt"):
        if row[0] != "words":
            continue
        w = np.array([[int(row[1], 16)]], dtype=np.uint32)
        assert O.unpack_int4(w, 8)[0].tolist() == [int(v) for v in row[2:]]


def test_single_nibble_positions():
    """A single set nibble at bit 4*i of word j dequantises only element 8j+i."""
    for j in range(3):
        for i in range(8):
            w = np.zeros((1, 3), dtype=np.uint32)
            w[0, j] = np.uint32(5) << np.uint32(4 * i)
            q = O.unpack_int4(w, 24)[0]
            expect = np.zeros(24, dtype=np.uint8)
            expect[8 * j + i] = 5
            assert np.array_equal(q, expect)


def test_group_sum_hand_example():
    """Hand-worked group: q_i = i mod 16, s = 2^-7, b = -2^-4, x = 1 -> -0.125."""
    row = [r for r in _lines("int4_words.txt") if r[0] == "groupsum"][0]
    g, s, b, expect = int(row[1]), float(row[2]), float(row[3]), float(row[4])
    q = (np.arange(g) % 16).reshape(1, g)
    W = O.dequant(G.pack_int4(q), bf([[s]]), bf([[b]]), g)
    assert W.sum() == expect


def test_group_scale_applies_to_its_own_columns():
    """Groups run along the input axis: columns [g*j, g*(j+1)) use scale j."""
    g, n_in = 8, 32
    q = np.full((2, n_in), 9)                     # q - 8 = 1 everywhere
    s = np.array([[1, 2, 4, 8], [0.5, 0.25, 0.125, 16]], dtype=np.float32)
    W = O.dequant(G.pack_int4(q), bf(s), bf(-8 * s), g)
    assert np.array_equal(W, np.repeat(s.astype(np.float64), g, axis=1))


def test_dequant_exact_in_fp64():
    """W = s*q + b agrees with the exact fp64 value rounded to fp32 for every
    code and sampled bf16 scales (s*q is exact: 8 x 4 significant bits)."""
    rng = np.random.default_rng(1)
    s = G.to_bf16_bits(rng.uniform(0.005, 0.02, size=(16, 1)).astype(np.float32))
    b = G.to_bf16_bits(rng.normal(0, 0.1, size=(16, 1)).astype(np.float32))
    q = np.tile(np.arange(16), (16, 1))
    W = O.dequant(G.pack_int4(q), s, b, 16)
    sf, bf_ = O.bf16_to_f64(s), O.bf16_to_f64(b)
    exact32 = (sf * q + bf_).astype(np.float32)
    assert np.array_equal(W.astype(np.float32), exact32)


def test_bundle_bytes_match_printed_sizes():
    """Pins the storage format (4 bits per weight + a bf16 scale and bias per
    group of 64) against the expert sizes the paper prints for its 35B tier."""
    rows = {r[0]: r[1:] for r in _lines("bundle_bytes.txt")}
    d, I, g, E, L, K = (int(v) for v in rows["shape"])
    shape = G.MoEShape(d, E, I, K, g, 0, 0.0, 0)
    per_expert = sum(a.nbytes for a in G.expert_tensors(shape, 0, 0, 0).values())
    got = {
        "per_expert_MB": per_expert / 1e6,
        "per_layer_MB": per_expert * E / 1e6,
        "all_layers_GB": per_expert * E * L / 1e9,
        "all_layers_GiB": per_expert * E * L / 2**30,
        "k_layer_MB": per_expert * K / 1e6,
    }
    for key, val in got.items():
        want, tol = float(rows[key][0]), float(rows[key][1])
        assert abs(val - want) <= tol * want, (key, val, want)


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 1.0 + 2**-8 + 2**-20, 3.0])
    want = np.array([1.0, 1.0 + 2**-6, -1.0, 1.0 + 2**-7, 3.0])
    assert np.array_equal(O.bf16_to_f64(O.f64_to_bf16_bits(vals)), want)


# ---------------------------------------------------------------- activations
def test_gelu_erf_values():
    for z, want in ((float(a), float(b)) for a, b in _lines("gelu_erf.txt")):
        assert abs(float(O.gelu_erf(z)) - want) <= 1e-14 * max(1.0, abs(want))
    z = np.linspace(-6, 6, 97)
    assert np.allclose(O.gelu_erf(z) - O.gelu_erf(-z), z, rtol=0, atol=1e-14)


def test_silu_closed_forms():
    """silu(ln 3) = 0.75 ln 3; silu(z) - silu(-z) = z; silu(0) = 0."""
    assert abs(float(O.silu(math.log(3.0))) - 0.75 * math.log(3.0)) < 1e-15
    z = np.linspace(-30, 30, 121)
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-12)
    assert float(O.silu(0.0)) == 0.0


# ---------------------------------------------------------------- expert FFN
def _structured_expert(d=64, I=32, g=32):
    """Expert whose every projection row has exactly one nonzero weight:
    q = 8 and b = -8 s everywhere except q = 8 + a at one column per row.
    Returns arrays and the column/value maps for the closed form."""
    def proj(rows, cols, col_of, a_of, s_grp):
        q = np.full((rows, cols), 8)
        for r in range(rows):
            q[r, col_of[r]] = 8 + a_of[r]
        s = np.tile(np.asarray(s_grp, dtype=np.float32), (rows, 1))
        return G.pack_int4(q), bf(s), bf(-8 * s)

    cg = [(5 * i + 3) % d for i in range(I)]
    ag = [((i % 7) - 3) or 2 for i in range(I)]
    cu = [(11 * i + 1) % d for i in range(I)]
    au = [((i % 5) - 2) or -3 for i in range(I)]
    cd = [(7 * o + 2) % I for o in range(d)]
    ad = [((o % 9) - 4) or 5 for o in range(d)]
    sg = [2**-3, 2**-2]                # d/g = 2 groups per gate/up row
    su = [2**-2, 2**-4]
    sd = [2**-1]                       # I/g = 1 group per down row
    ex = {}
    ex["gate_q"], ex["gate_s"], ex["gate_b"] = proj(I, d, cg, ag, sg)
    ex["up_q"], ex["up_s"], ex["up_b"] = proj(I, d, cu, au, su)
    ex["down_q"], ex["down_s"], ex["down_b"] = proj(d, I, cd, ad, sd)
    return ex, (cg, ag, sg, cu, au, su, cd, ad, sd)


def test_expert_ffn_structured_closed_form():
    """One nonzero weight per row: G_i = s*a_i*x[c_i] (its group's scale),
    U_i likewise, h = silu(G)*U, D_o = s*a_o*h[c_o].  Pins row/column
    orientation, group indexing and the gate/up roles of SwiGLU."""
    d, I, g = 64, 32, 32
    ex, (cg, ag, sg, cu, au, su, cd, ad, sd) = _structured_expert(d, I, g)
    x = np.array([(j - 32) / 8.0 for j in range(d)])
    D = O.expert_ffn(ex, x, g)
    Gv = [sg[cg[i] // g] * ag[i] * x[cg[i]] for i in range(I)]
    Uv = [su[cu[i] // g] * au[i] * x[cu[i]] for i in range(I)]
    h = [Gv[i] / (1.0 + math.exp(-Gv[i])) * Uv[i] for i in range(I)]
    want = [sd[0] * ad[o] * h[cd[o]] for o in range(d)]
    assert np.allclose(D, want, rtol=1e-13, atol=1e-15)


def _tiny_layer(seed=0, shape=G.TINY):
    experts = {e: G.expert_tensors(shape, seed, 0, e) for e in range(shape.n_experts)}
    lora = {e: G.lora_tensors(shape, seed, 0, e) for e in range(shape.n_experts)}
    return experts, lora


def test_lora_zero_b_is_bit_identical():
    """B = 0 makes the delta exactly zero: output identical to no adapter."""
    shape = G.TINY
    experts, lora = _tiny_layer()
    zero_b = {e: {**l, "b_gate": np.zeros_like(l["b_gate"]), "b_up": np.zeros_like(l["b_up"]),
                  "b_down": np.zeros_like(l["b_down"])} for e, l in lora.items()}
    x = G.hidden(shape, 0)
    ids, w = np.array([3, 0, 7, 12]), np.array([0.4, 0.3, 0.2, 0.1])
    y0 = O.moe_layer(experts, ids, w, x, shape.group)
    y1 = O.moe_layer(experts, ids, w, x, shape.group, zero_b, 2.0)
    assert np.array_equal(y0, y1)


def test_lora_unmerged_equals_merged():
    """Unmerged W x + (a/r) B (A x) equals (W + (a/r) B A) x  (associativity)."""
    shape = G.TINY
    experts, lora = _tiny_layer()
    x = O.bf16_to_f64(G.hidden(shape, 0))
    ex, lo = experts[5], lora[5]
    W = O.dequant(ex["gate_q"], ex["gate_s"], ex["gate_b"], shape.group)
    A, B = O.bf16_to_f64(lo["a_gate"]), O.bf16_to_f64(lo["b_gate"])
    merged = (W + (16.0 / 8.0) * (B @ A)) @ x
    unmerged = O.lora_proj(W, x, lo["a_gate"], lo["b_gate"], shape.lora_alpha / shape.lora_rank)
    assert np.linalg.norm(merged - unmerged) <= 1e-12 * np.linalg.norm(merged)
    assert np.linalg.norm(unmerged - W @ x) > 1e-3 * np.linalg.norm(W @ x)   # delta is not negligible


@pytest.mark.parametrize("shape,rms", [(G.TINY, 1.13e-3), (G.QWEN3_MOE, 1.60e-3)])
def test_lora_delta_rms_closed_form(shape, rms):
    """Weight-level delta (a/r) B A has RMS (a/r) sqrt(r) sA sB: 1.13e-3 for
    r=8, a=16 and 1.60e-3 for r=16, a=32 - the "RMS 1e-3" scale of the
    paper's §3.3.  Measured through the oracle on unit vectors."""
    lo = G.lora_tensors(shape, 0, 0, 0)
    n_in = shape.d_model
    cols = np.eye(n_in)[:, :256]
    delta = O.lora_proj(np.zeros((shape.d_inter, n_in)), cols, lo["a_gate"], lo["b_gate"],
                        shape.lora_alpha / shape.lora_rank)
    got = float(np.sqrt(np.mean(delta**2)))
    assert abs(got - rms) < 0.06 * rms, got


def test_moe_combine_uniform_equals_dense_mean():
    """K = E with all logits equal: w = 1/E and y = mean over all experts."""
    shape = G.TINY
    experts, lora = _tiny_layer()
    x = G.hidden(shape, 3)
    ids, w = O.softmax_topk(np.zeros(shape.n_experts), shape.n_experts)
    assert np.allclose(w, 1.0 / shape.n_experts, rtol=0, atol=1e-15)
    y = O.moe_layer(experts, ids, w, x, shape.group, lora, 2.0)
    xf = O.bf16_to_f64(x)
    dense = np.mean([O.expert_ffn(experts[e], xf, shape.group, lora[e], 2.0)
                     for e in range(shape.n_experts)], axis=0)
    assert np.linalg.norm(y - dense) <= 1e-12 * np.linalg.norm(dense)


def test_moe_weight_pairs_with_its_id():
    """A one-hot weight vector selects exactly the expert listed at that
    position: w = e_k gives y = FFN_{ids[k]}(x)."""
    shape = G.TINY
    experts, lora = _tiny_layer()
    x = G.hidden(shape, 4)
    ids = np.array([6, 2, 11, 0])
    for k in range(4):
        w = np.zeros(4)
        w[k] = 1.0
        y = O.moe_layer(experts, ids, w, x, shape.group, lora, 2.0)
        want = O.expert_ffn(experts[ids[k]], O.bf16_to_f64(x), shape.group, lora[ids[k]], 2.0)
        assert np.array_equal(y, want)


def test_moe_linear_in_weights():
    """y is linear in the routing weights: w -> 2w doubles y."""
    shape = G.TINY
    experts, lora = _tiny_layer()
    x = G.hidden(shape, 4)
    ids, w = np.array([1, 2, 3, 4]), np.array([0.1, 0.2, 0.3, 0.4])
    y1 = O.moe_layer(experts, ids, w, x, shape.group, lora, 2.0)
    y2 = O.moe_layer(experts, ids, 2 * w, x, shape.group, lora, 2.0)
    assert np.allclose(y2, 2 * y1, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- routing
def test_topk_brute_force():
    """For E <= 16 the chosen set is the unique maximiser of the summed
    logits over all C(E, K) subsets, listed by descending logit."""
    rng = np.random.default_rng(7)
    for E, K in ((8, 2), (12, 4), (16, 4), (16, 8), (10, 1)):
        for _ in range(20):
            l = rng.normal(size=E)
            ids, w = O.softmax_topk(l, K)
            best = max(itertools.combinations(range(E), K), key=lambda S: sum(l[list(S)]))
            assert sorted(ids.tolist()) == sorted(best)
            assert all(l[ids[i]] > l[ids[i + 1]] for i in range(K - 1))
            assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)


def test_topk_special_cases():
    rng = np.random.default_rng(8)
    l = rng.normal(size=16)
    assert O.softmax_topk(l, 1)[0][0] == np.argmax(l)
    ids, w = O.softmax_topk(l, 16)
    assert np.allclose(w, scipy.special.softmax(l)[ids], rtol=1e-14, atol=0)
    ids2, w2 = O.softmax_topk(l + 17.25, 4)
    ids1, w1 = O.softmax_topk(l, 4)
    assert np.array_equal(ids1, ids2) and np.allclose(w1, w2, rtol=1e-12)
    # ties go to the lower index
    ids, w = O.softmax_topk(np.array([0.5, 1.0, 1.0, 0.0, 1.0]), 2)
    assert ids.tolist() == [1, 2] and np.allclose(w, 0.5)


def test_topk_weights_ignore_unselected_logits():
    """Renormalisation over the selected set: lowering a non-selected logit
    leaves the weights unchanged (the full-softmax normaliser cancels)."""
    rng = np.random.default_rng(9)
    l = rng.normal(size=16)
    ids, w = O.softmax_topk(l, 4)
    other = [e for e in range(16) if e not in ids][0]
    l2 = l.copy()
    l2[other] -= 5.0
    ids2, w2 = O.softmax_topk(l2, 4)
    assert np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- prerouter
def test_prerouter_toy_feature_layout():
    rows = {r[0]: r[1:] for r in _lines("prerouter_toy.txt")}
    d, E = int(rows["d_model"][0]), int(rows["n_experts"][0])
    x = bf(np.arange(1, d + 1) / 8.0)
    f = O.prerouter_feature(x, [int(v) for v in rows["ids_now"]],
                            [int(v) for v in rows["ids_prev"]], E)
    assert f.shape == (d + 2 * E,)
    assert np.array_equal(f[:d], np.arange(1, d + 1) / 8.0)
    ones = sorted(int(v) for v in rows["ones"])
    assert np.flatnonzero(f[d:]).tolist() == [i - d for i in ones] and np.all(f[ones] == 1.0)


def _head(shape, seed=0):
    return G.head_tensors(shape, seed, 0)


def test_prerouter_warm_start_identity():
    """fc2 = 0 and b2 = 0: logits reduce to the residual l(x); with l set to
    the next layer's router matrix they equal that router's logits exactly."""
    shape = G.TINY
    rng = np.random.default_rng(2)
    vals = (rng.integers(-64, 64, size=(shape.n_experts, shape.d_model)) / 256.0).astype(np.float32)
    head = dict(_head(shape))
    head["w2"] = np.zeros_like(head["w2"])
    head["b2"] = None
    head["wl"] = vals.astype(np.float16)          # exact in fp16 and bf16
    x = G.hidden(shape, 5)
    got = O.prerouter_logits(head, x, [0, 1, 2, 3], [4, 5, 6, 7], shape.n_experts)
    assert np.array_equal(got, O.router_logits(bf(vals), x))


def test_prerouter_gather_form_and_block_order():
    """fc1 on the dense feature equals W1x x + sum of the 'now' block rows of
    w1oh at this token's ids + the 'prev' block rows (offset E) + b1; with
    the residual off the logits are fc2(gelu(.)) + b2."""
    shape = G.TINY
    E = shape.n_experts
    head = dict(_head(shape))
    x = G.hidden(shape, 6)
    now, prev = [2, 9, 4, 15], [1, 2, 3, 0]
    W1oh = head["w1oh"].astype(np.float64)
    z1 = (head["w1x"].astype(np.float64) @ O.bf16_to_f64(x) + W1oh[now].sum(0)
          + W1oh[[E + e for e in prev]].sum(0) + head["b1"].astype(np.float64))
    a = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z1])
    want = head["w2"].astype(np.float64) @ a + head["b2"].astype(np.float64)
    head["wl"] = None
    got = O.prerouter_logits(head, x, now, prev, E)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    # swapping the two blocks changes the prediction input
    assert not np.allclose(O.prerouter_logits(head, x, prev, now, E), got)
    # no previous token: the prev block is all zeros
    z1b = z1 - W1oh[[E + e for e in prev]].sum(0)
    ab = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z1b])
    wantb = head["w2"].astype(np.float64) @ ab + head["b2"].astype(np.float64)
    assert np.allclose(O.prerouter_logits(head, x, now, None, E), wantb, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- stack
def test_rmsnorm_closed_form():
    h = np.array([3.0, 4.0, 0.0, 0.0])
    assert np.allclose(O.rmsnorm(h, 0.0), [1.2, 1.6, 0.0, 0.0], rtol=1e-15, atol=0)
    assert np.allclose(O.rmsnorm(h, 1e-6), np.array([3, 4, 0, 0]) / math.sqrt(6.25 + 1e-6),
                       rtol=1e-15, atol=0)
    assert np.array_equal(O.rmsnorm(np.zeros(4)), np.zeros(4))


class _ZeroLayer:
    """A layer whose experts are all zero (q = 8, b = -8 s)."""

    def __init__(self, shape, seed, L):
        self.shape, self.seed, self.L = shape, seed, L
        self.router = G.router_weight(shape, seed, L)
        self.head = G.head_tensors(shape, seed, L)

    def expert(self, e):
        ex = G.expert_tensors(self.shape, self.seed, self.L, e)
        for p in ("gate", "up", "down"):
            ex[p + "_q"] = np.full_like(ex[p + "_q"], 0x88888888)
        return ex

    def lora(self, e):
        lo = G.lora_tensors(self.shape, self.seed, self.L, e)
        return {k: (np.zeros_like(v) if k.startswith("b_") else v) for k, v in lo.items()}


def test_stack_zero_experts_is_identity_residual():
    """All-zero experts give y = 0, so the residual block returns h itself
    (pins h' = h + y rather than x + y), and routing still follows the rules:
    router at t = 0, the committed prediction at t > 0 on consumer layers."""
    shape = G.TINY
    layers = [_ZeroLayer(shape, 0, L) for L in range(10)]
    h0 = G.stack_hidden(shape, 0, 0)
    owners, consumers = range(2, 8), range(3, 9)
    h, res, committed, executed = O.stack_step(layers, h0, 0, {}, {}, shape, owners, consumers)
    assert np.array_equal(h, h0)
    assert sorted(committed) == list(range(3, 9))
    for L, r in enumerate(res):
        assert np.array_equal(r["h_next"], h0) and np.all(r["y"] == 0)
        assert r["router_logits"] is not None
    h1 = G.stack_hidden(shape, 0, 1)
    h, res1, committed1, _ = O.stack_step(layers, h1, 1, committed, executed, shape, owners, consumers)
    for L in range(10):
        if L in consumers:
            assert res1[L]["router_logits"] is None
            assert np.array_equal(res1[L]["ids"], committed[L][0])
        else:
            assert res1[L]["router_logits"] is not None


# ---------------------------------------------------------------- slot pool
def _lru_cases():
    cases, cur = {}, None
    for row in _lines("lru_trace.txt"):
        if row[0] == "case":
            cur = cases.setdefault(row[1], {"n": int(row[2]), "ev": []})
        else:
            cur["ev"].append(row)
    return cases


def test_lru_hand_traces():
    for name, case in _lru_cases().items():
        events, sets, want = [], {}, []
        for row in case["ev"]:
            L, t = int(row[1]), int(row[2])
            if row[0] == "use":
                events.append(("use", L, t))
                continue
            bar = row.index("|")
            bar2 = row.index("|", bar + 1)
            sets[(L, t)] = [int(v) for v in row[3:bar]]
            want.append(([int(v) for v in row[bar + 1:bar2]], [v == "1" for v in row[bar2 + 1:]]))
            events.append(("req", L, t))
        recs, tot = O.lru_replay(events, lambda L, t: sets[(L, t)], case["n"])
        assert [(r["slots"], r["hit"]) for r in recs] == want, name


def test_lru_all_pinned_raises():
    with pytest.raises(O.NoSlotError):
        O.lru_replay([("req", 0, 0), ("req", 0, 1)], lambda L, t: [[1, 2], [3]][t], 2)


def test_lru_invariants_on_trace():
    """Over a Zipf trace: every pending (layer, id) maps to a slot holding it,
    no slot holds two bundles, hits + misses = touches, and with room for
    every bundle the misses equal the distinct (layer, id) count."""
    L, T, E, K = 12, 20, 16, 4
    trace = G.zipf_trace(E, K, L, T + 1, seed=3, keep_p=0.1)
    ev = O.canonical_requests(T, L, owners=range(2, 10), consumers=range(3, 11))
    recs, tot = O.lru_replay(ev, lambda l, t: trace[t, l], 40)
    assert tot["hits"] + tot["misses"] == tot["touches"] == sum(len(r["ids"]) for r in recs)
    holder = {}
    for r in recs:
        for e, s in zip(r["ids"], r["slots"]):
            holder[s] = (r["L"], e)
        assert len(set(r["slots"])) == len(r["slots"])
    recs2, tot2 = O.lru_replay(ev, lambda l, t: trace[t, l], L * E)
    distinct = {(r["L"], e) for r in recs2 for e in r["ids"]}
    assert tot2["misses"] == len(distinct)


def test_canonical_requests_order():
    """Owner layer L requests (L+1, t+1) right after using (L, t); consumer
    layers request nothing themselves after t = 0."""
    ev = O.canonical_requests(2, 4, owners=range(1, 3), consumers=range(2, 4))
    assert ev[:8] == [("req", 0, 0), ("use", 0, 0), ("req", 1, 0), ("use", 1, 0), ("req", 2, 1),
                      ("req", 2, 0), ("use", 2, 0), ("req", 3, 1)]
    assert ("req", 2, 1) in ev and ("req", 3, 1) in ev
    assert [e for e in ev if e[2] == 1 and e[0] == "req" and e[1] >= 2] == [("req", 2, 1), ("req", 3, 1)]


def test_canonical_requests_heads_at_end():
    """Batched heads: a step's predicted sets are requested after its last
    layer, in owner order; the per-layer events are otherwise unchanged."""
    ev = O.canonical_requests(2, 4, owners=range(1, 3), consumers=range(2, 4), heads_at_end=True)
    assert ev[:10] == [("req", 0, 0), ("use", 0, 0), ("req", 1, 0), ("use", 1, 0),
                       ("req", 2, 0), ("use", 2, 0), ("req", 3, 0), ("use", 3, 0),
                       ("req", 2, 1), ("req", 3, 1)]
    # step 1: layers 2, 3 consume the sets requested at the end of step 0
    assert ev[10:16] == [("req", 0, 1), ("use", 0, 1), ("req", 1, 1), ("use", 1, 1),
                         ("use", 2, 1), ("use", 3, 1)]
    # every request is used exactly once before the end, except the last
    # step's predictions
    reqs = [e[1:] for e in ev if e[0] == "req"]
    uses = [e[1:] for e in ev if e[0] == "use"]
    assert sorted(set(reqs) - set(uses)) == [(2, 2), (3, 2)]
    assert sorted(uses) == sorted(set(uses))


def test_lru_on_demand_order_never_pins_two_sets():
    """With no consumers every set is requested right before its use, so at
    most one set is pinned: a pool of exactly K slots never runs out, and
    with K slots every request of a new layer misses entirely."""
    E, K, L, T = 16, 4, 5, 6
    trace = G.zipf_trace(E, K, L, T, seed=5, keep_p=0.2)
    ev = O.canonical_requests(T, L, owners=range(0), consumers=range(0))
    recs, tot = O.lru_replay(ev, lambda l, t: trace[t, l], K)
    assert len(recs) == L * T
    for r in recs:
        assert sorted(r["slots"]) == list(range(K))
        if L > 1:
            assert not any(r["hit"])


def test_softmax_at_closed_forms():
    """w_i / w_j = exp(l_i - l_j); sum w = 1; shift invariance; on the top-K
    ids it reproduces the committed weights."""
    rng = np.random.default_rng(11)
    l = rng.normal(size=32)
    ids = np.array([5, 17, 2, 30])
    w = O.softmax_at(l, ids)
    assert abs(w.sum() - 1.0) < 1e-15
    for i in range(4):
        for j in range(4):
            assert abs(w[i] / w[j] - math.exp(l[ids[i]] - l[ids[j]])) < 1e-12 * max(1, w[i] / w[j])
    assert np.allclose(O.softmax_at(l + 123.0, ids), w, rtol=1e-12, atol=0)
    tid, tw = O.softmax_topk(l, 4)
    assert np.allclose(O.softmax_at(l, tid), tw, rtol=1e-14, atol=0)
    # a single id gets weight 1
    assert O.softmax_at(l, [7])[0] == 1.0


# ---------------------------------------------------------------- grouped
def test_grouped_is_per_token():
    shape = G.TINY
    experts, lora = _tiny_layer()
    ids, w = G.grouped_routing(shape.n_experts, 4, 3, seed=1)
    x = G.hidden(shape, 9, n=3)
    y = O.grouped_layer(experts, ids, w, x, shape.group, lora, 2.0)
    for j in range(3):
        assert np.array_equal(y[j], O.moe_layer(experts, ids[j], w[j], x[j], shape.group, lora, 2.0))


def test_bf16_rounding_check_accepts_only_midpoint_flips():
    """The GPU-vs-oracle rounding criterion: a flip is accepted only at a
    near-midpoint exact value, between adjacent bf16 numbers."""
    from tests.layer_setup import check_bf16_rounding
    one = O.f64_to_bf16_bits(np.array([1.0]))[0]
    step = 2.0 ** -7
    # exact value just below the midpoint 1 + step/2: RNE gives 1.0; 1+step accepted
    e = np.array([1.0 + step / 2 - 1e-9])
    assert check_bf16_rounding(np.array([one + 1], np.uint16), e) == 1
    # far from the midpoint: the other neighbour is rejected
    with pytest.raises(AssertionError):
        check_bf16_rounding(np.array([one + 1], np.uint16), np.array([1.0 + step / 8]))
    # two steps away: rejected
    with pytest.raises(AssertionError):
        check_bf16_rounding(np.array([one + 2], np.uint16), e)
    assert check_bf16_rounding(np.array([one], np.uint16), np.array([1.0])) == 0
