"""GPU parity of merge-and-requantise (edge0_merge_requant, [Edge0] §3.3 and
its footnote 2) against the oracle: the merged bundle's codes, scales and
biases for gate, up and down (down in its tiled layout), the weight-level
retention per projection, and the merged bundle used by the layer kernel
against the oracle's layer on the oracle's requantised weights."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, DeviceLayer, rel_l2

pytestmark = pytest.mark.gpu

CODE_GAP = 1e-4  # codes compared exactly unless (w' - b') / s' is this close to k + 1/2
BF16_GAP = 1e-6  # scales/biases exactly unless the exact value is this close (relative) to a bf16 midpoint


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _unpack_rows(words, n_in):
    return O.unpack_int4(words, n_in)


def _down_codes(buf_u32, d, I):
    """Logical [d][I] codes from the tiled down array [d/64][I/32][64][4]."""
    t = buf_u32.reshape(d // 64, I // 32, 64, 4)
    words = t.transpose(0, 2, 1, 3).reshape(d, I // 8)  # row o: its words in input order
    return O.unpack_int4(words, I)


def _near_mid(exact):
    """True where the exact value is within BF16_GAP of a bf16 rounding
    midpoint: the midpoint between its rounding and the bf16 neighbour on the
    exact value's side (for a negative number one more in the bit pattern is
    further from zero)."""
    b = O.f64_to_bf16_bits(exact).astype(np.int32)
    v = O.bf16_to_f64(b.astype(np.uint16))
    up, dn = (O.bf16_to_f64(((b + k) & 0xFFFF).astype(np.uint16)) for k in (1, -1))
    with np.errstate(invalid="ignore"):
        nb = np.where(np.sign(up - v) == np.sign(exact - v), up, dn)
        mid = (v + nb) / 2
        return np.abs(exact - mid) <= BF16_GAP * np.abs(exact) + 1e-300


def _check_projection(q_gpu, s_gpu, b_gpu, words, s_bits, b_bits, A, B, scale, g):
    (q_o, s_o, b_o), actual, ret = O.merge_requant(words, s_bits, b_bits, A, B, scale, g)
    W = O.dequant(words, s_bits, b_bits, g) + O.lora_delta(A, B, scale)
    out_dim, n_in = W.shape
    Wg = W.reshape(out_dim, n_in // g, g)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    waive_g = _near_mid((hi - lo) / 15.0) | _near_mid(lo)
    same = (s_gpu == s_o) & (b_gpu == b_o)
    assert np.all(same | waive_g), np.argwhere(~(same | waive_g))[:4]
    sv = O.bf16_to_f64(s_o).repeat(g, axis=1)
    bv = O.bf16_to_f64(b_o).repeat(g, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(sv > 0, (W - bv) / sv, 0.0)
    near = np.abs(u - np.floor(u) - 0.5) < CODE_GAP
    ok_el = (q_gpu == q_o) | near | ~same.repeat(g, axis=1)
    assert ok_el.all(), np.argwhere(~ok_el)[:4]
    return ret, int((~same).sum()), int(near.sum())


@pytest.mark.parametrize("name,S,experts", [("tiny", G.TINY, range(16)),
                                           ("qwen3moe", G.QWEN3_MOE, (0, 77))])
def test_merge_requant_parity(torch_cuda, name, S, experts):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    lay = DeviceLayer(S, seed=6, layer=2)
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    lay0 = E.edge0_bundle_layout_of(sh0)
    dst = torch.zeros(int(lay0.bytes), dtype=torch.uint8, device="cuda")
    stats = torch.zeros(6, dtype=torch.float64, device="cuda")
    ws = None
    d, I, g = S.d_model, S.d_inter, S.group
    scale = S.lora_alpha / S.lora_rank
    for e in experts:
        print(f"[merge] {name} expert {e}", flush=True)
        stats.fill_(float("nan"))  # every call must write all six figures
        ws = E.edge0_merge_requant(lay.sh, lay.pool.slot_ptr(e), dst, stats, ws)
        torch.cuda.synchronize()
        buf = dst.cpu().numpy()
        st = stats.cpu().numpy()
        ex, lo = lay.experts[e], lay.loras[e]

        def arr(off, n, dt):
            return np.frombuffer(buf[off:off + n * np.dtype(dt).itemsize].tobytes(), dtype=dt)
        for p, (proj, n_out, n_in) in enumerate((("gate", I, d), ("up", I, d), ("down", d, I))):
            qo = getattr(lay0, proj + "_q")
            if proj == "down":
                q_gpu = _down_codes(arr(qo, d * I // 8, np.uint32), d, I)
                s_gpu = arr(lay0.down_s, (I // g) * d, np.uint16).reshape(I // g, d).T
                b_gpu = arr(lay0.down_b, (I // g) * d, np.uint16).reshape(I // g, d).T
            else:
                q_gpu = _unpack_rows(arr(qo, n_out * n_in // 8, np.uint32).reshape(n_out, n_in // 8), n_in)
                s_gpu = arr(getattr(lay0, proj + "_s"), n_out * (n_in // g), np.uint16).reshape(n_out, -1)
                b_gpu = arr(getattr(lay0, proj + "_b"), n_out * (n_in // g), np.uint16).reshape(n_out, -1)
            ret, n_waived_g, n_near = _check_projection(
                q_gpu, s_gpu, b_gpu, ex[proj + "_q"], ex[proj + "_s"], ex[proj + "_b"],
                lo["a_" + proj], lo["b_" + proj], scale, g)
            ret_gpu = st[2 * p] / st[2 * p + 1]
            assert abs(ret_gpu - ret) <= 1e-3 * max(1.0, abs(ret)) + 1e-4, (proj, ret_gpu, ret)
            print(f"[merge] {name} e{e} {proj}: retention {ret_gpu:.4f} (oracle {ret:.4f}), "
                  f"{n_waived_g} groups and {n_near} codes at near-ties")


# Group widths and ranks beyond the two model shapes: groups of 128, 96 and
# 32 inputs (8, 6 and 2 blocks of 16 inputs per unit of the matrix-core
# kernel), groups of 256 (the one-thread-per-group kernel), rank 0
# (no delta: the stats stay 0 and the merge is the base requantised), and
# ranks 8, 32 and 64 (one, one and two rank chunks of the matrix-core
# product; 64 at 128 inputs is the kernel's largest register set).
WIDTH_CASES = [
    ("g128_r32", G.MoEShape(512, 2, 256, 1, 128, 32, 64.0, 64), True),
    ("g96_r64", G.MoEShape(6144, 2, 192, 1, 96, 64, 128.0, 64), True),
    ("g256_r16", G.MoEShape(512, 2, 256, 1, 256, 16, 32.0, 64), True),
    ("g64_r0", G.MoEShape(256, 2, 128, 1, 64, 8, 16.0, 64), False),
    ("g32_r64", G.MoEShape(256, 2, 128, 1, 32, 64, 128.0, 64), True),
    ("g128_r64", G.MoEShape(512, 2, 256, 1, 128, 64, 128.0, 64), True),
    ("g64_r8", G.MoEShape(512, 2, 256, 1, 64, 8, 16.0, 64), True),
]


@pytest.mark.parametrize("name,S,lora", WIDTH_CASES, ids=[c[0] for c in WIDTH_CASES])
def test_merge_requant_group_widths(torch_cuda, name, S, lora):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    lay = DeviceLayer(S, seed=9, layer=1, lora=lora)
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    lay0 = E.edge0_bundle_layout_of(sh0)
    d, I, g = S.d_model, S.d_inter, S.group
    r = S.lora_rank if lora else 0
    scale = S.lora_alpha / S.lora_rank if lora else 0.0
    stats = torch.zeros(6, dtype=torch.float64, device="cuda")
    ws = None
    for e in range(S.n_experts):
        print(f"[merge] {name} expert {e}", flush=True)
        dst = torch.full((int(lay0.bytes),), 0xA5, dtype=torch.uint8, device="cuda")
        stats.fill_(float("nan"))  # every call must write all six figures
        ws = E.edge0_merge_requant(lay.sh, lay.pool.slot_ptr(e), dst, stats, ws)
        torch.cuda.synchronize()
        buf = dst.cpu().numpy()
        st = stats.cpu().numpy()
        ex = lay.experts[e]

        def arr(off, n, dt):
            return np.frombuffer(buf[off:off + n * np.dtype(dt).itemsize].tobytes(), dtype=dt)
        for p, (proj, n_out, n_in) in enumerate((("gate", I, d), ("up", I, d), ("down", d, I))):
            qo = getattr(lay0, proj + "_q")
            if proj == "down":
                q_gpu = _down_codes(arr(qo, d * I // 8, np.uint32), d, I)
                s_gpu = arr(lay0.down_s, (I // g) * d, np.uint16).reshape(I // g, d).T
                b_gpu = arr(lay0.down_b, (I // g) * d, np.uint16).reshape(I // g, d).T
            else:
                q_gpu = _unpack_rows(arr(qo, n_out * n_in // 8, np.uint32).reshape(n_out, n_in // 8), n_in)
                s_gpu = arr(getattr(lay0, proj + "_s"), n_out * (n_in // g), np.uint16).reshape(n_out, -1)
                b_gpu = arr(getattr(lay0, proj + "_b"), n_out * (n_in // g), np.uint16).reshape(n_out, -1)
            if lora:
                A, B = lay.loras[e]["a_" + proj], lay.loras[e]["b_" + proj]
            else:
                A, B = np.zeros((0, n_in), np.uint16), np.zeros((n_out, 0), np.uint16)
            ret, n_waived_g, n_near = _check_projection(
                q_gpu, s_gpu, b_gpu, ex[proj + "_q"], ex[proj + "_s"], ex[proj + "_b"],
                A, B, scale, g)
            if r == 0:
                assert st[2 * p] == 0.0 and st[2 * p + 1] == 0.0, (proj, st)
            else:
                ret_gpu = st[2 * p] / st[2 * p + 1]
                assert abs(ret_gpu - ret) <= 1e-3 * max(1.0, abs(ret)) + 1e-4, (proj, ret_gpu, ret)
            print(f"[merge] {name} e{e} {proj}: {n_waived_g} groups and {n_near} codes at near-ties")

def test_merged_bundle_runs_in_the_layer(torch_cuda):
    """Merged bundles (LoRA-free layout) in a pool of their own through
    edge0_moe_layer with lora_rank 0, against the oracle's layer on the
    oracle's requantised weights."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = G.TINY
    lay = DeviceLayer(S, seed=7, layer=0)
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    bb0 = int(E.edge0_bundle_layout_of(sh0).bytes)
    pool_mem = torch.zeros(S.n_experts * bb0, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(6, dtype=torch.float64, device="cuda")
    merged = {}
    scale = S.lora_alpha / S.lora_rank
    for e in range(S.n_experts):
        E.edge0_merge_requant(lay.sh, lay.pool.slot_ptr(e), pool_mem[e * bb0:(e + 1) * bb0], stats)
        ex, lo = lay.experts[e], lay.loras[e]
        m = {}
        for proj, n_in in (("gate", S.d_model), ("up", S.d_model), ("down", S.d_inter)):
            (q, s2, b2), _, _ = O.merge_requant(ex[proj + "_q"], ex[proj + "_s"], ex[proj + "_b"],
                                                lo["a_" + proj], lo["b_" + proj], scale, S.group)
            qq = q.astype(np.uint32).reshape(q.shape[0], n_in // 8, 8) << (4 * np.arange(8, dtype=np.uint32))
            m[proj + "_q"] = np.bitwise_or.reduce(qq, axis=2).astype(np.uint32)
            m[proj + "_s"], m[proj + "_b"] = s2, b2
        merged[e] = m
    torch.cuda.synchronize()
    pool = E.SlotPool(pool_mem.data_ptr(), bb0, S.n_experts)
    ws = E.new_workspace(sh0)
    for i in range(6):
        x = G.hidden(S, 300 + i)
        ids = np.random.default_rng(i).choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        w = np.full(S.top_k, 1.0 / S.top_k, np.float32)
        y = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
        E.edge0_moe_layer(sh0, pool, lay.table, torch.from_numpy(ids).cuda(),
                          torch.from_numpy(w).cuda(), to_device(x), y, ws)
        torch.cuda.synchronize()
        y_o = O.moe_layer(merged, ids, w.astype(np.float64), x, S.group)
        assert rel_l2(O.bf16_to_f64(y.cpu().numpy().view(np.uint16)), y_o) <= REL_L2_MAX


def test_output_retention_matches_oracle(torch_cuda):
    """The output-level retention 1 - |U - M| / |U - B| of 32 tiny-layer
    calls from the GPU's bf16 outputs (U with the LoRA, M on the merged
    bundles, B on the base) against the oracle's fp64 value on the same
    tokens; the bf16 rounding of the outputs allows 0.05."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = G.TINY
    lay = DeviceLayer(S, seed=8, layer=1)
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    bb0 = int(E.edge0_bundle_layout_of(sh0).bytes)
    pool_mem = torch.zeros(S.n_experts * bb0, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(6, dtype=torch.float64, device="cuda")
    scale = S.lora_alpha / S.lora_rank
    merged = {}
    for e in range(S.n_experts):
        E.edge0_merge_requant(lay.sh, lay.pool.slot_ptr(e), pool_mem[e * bb0:(e + 1) * bb0], stats)
        m = {}
        ex, lo = lay.experts[e], lay.loras[e]
        for proj, n_in in (("gate", S.d_model), ("up", S.d_model), ("down", S.d_inter)):
            (q, s2, b2), _, _ = O.merge_requant(ex[proj + "_q"], ex[proj + "_s"], ex[proj + "_b"],
                                                lo["a_" + proj], lo["b_" + proj], scale, S.group)
            qq = q.astype(np.uint32).reshape(q.shape[0], n_in // 8, 8) << (4 * np.arange(8, dtype=np.uint32))
            m[proj + "_q"] = np.bitwise_or.reduce(qq, axis=2).astype(np.uint32)
            m[proj + "_s"], m[proj + "_b"] = s2, b2
        merged[e] = m
    pool0 = E.SlotPool(pool_mem.data_ptr(), bb0, S.n_experts)
    ws = E.new_workspace(lay.sh)
    rng = np.random.default_rng(12)
    gU, gM, gB, oU, oM, oB = ([] for _ in range(6))
    for i in range(32):
        xb = G.hidden(S, 400 + i)
        ids = rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        w = np.full(S.top_k, 1.0 / S.top_k, np.float32)
        outs = []
        for shp, pool in ((lay.sh, lay.pool.pool), (sh0, pool0), (sh0, lay.pool.pool)):
            y = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
            E.edge0_moe_layer(shp, pool, lay.table, torch.from_numpy(ids).cuda(),
                              torch.from_numpy(w).cuda(), to_device(xb), y, ws)
            outs.append(y)
        torch.cuda.synchronize()
        for lst, y in zip((gU, gM, gB), outs):
            lst.append(O.bf16_to_f64(y.cpu().numpy().view(np.uint16)))
        w64 = w.astype(np.float64)
        oU.append(O.moe_layer(lay.experts, ids, w64, xb, S.group, lay.loras, scale))
        oM.append(O.moe_layer(merged, ids, w64, xb, S.group))
        oB.append(O.moe_layer(lay.experts, ids, w64, xb, S.group))
    r_gpu = O.layer_retention(np.stack(gU), np.stack(gM), np.stack(gB))
    r_or = O.layer_retention(np.stack(oU), np.stack(oM), np.stack(oB))
    print(f"[merge] output retention: GPU {r_gpu:.4f}, oracle {r_or:.4f}")
    assert abs(r_gpu - r_or) <= 0.05, (r_gpu, r_or)
