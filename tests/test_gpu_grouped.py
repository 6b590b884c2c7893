"""GPU parity of the grouped multi-token layer (edge0_moe_grouped) against
the oracle, which defines it token by token: y_j = sum_k w_jk FFN_{e_jk}(x_j).
Every token's output is compared (rel-L2 <= 2e-3), for the tiny shape
(many tokens per expert, several token batches, a ragged last batch) and the
Qwen3-MoE shape at K = 8 with 1, 4, 8, 16, 32 and 64 tokens and Zipf(1.1)
routing; the default path (MFMA tiles of up to 16 tokens for every expert
from 3 tokens per call on, GEMVs below), the GEMV path (at most 8 of an
expert's tokens per workgroup), the mixed path (tiles for experts with >= 16
tokens) and the tiles for every expert; determinism; reuse of the workspace
by a smaller call; one token alone equals its row of a grouped call; ids
repeated within a token; the empty call; invalid ids reported."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, DeviceLayer, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


_LAYERS = {}
# default, GEMV only, MFMA tiles from 16 tokens per expert, tiles for every
# expert
GEMV = 1
MFMA16 = 16 << 8
TILES = 1 << 8
FLAG_SETS = (0, GEMV, MFMA16, TILES)


def _layer(S):
    key = (S.d_model, S.top_k)
    if key not in _LAYERS:
        _LAYERS[key] = DeviceLayer(S, seed=2, layer=3)
    return _LAYERS[key]


def _call(lay, ids, w, x_bits, flags=0, ws=None):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    T = ids.shape[0]
    if ws is None:
        ws = E.new_grouped_workspace(lay.sh)
    y = torch.zeros((T, lay.S.d_model), dtype=torch.int16, device="cuda")
    E.edge0_moe_grouped(lay.sh, lay.pool.pool, lay.table, T, to_device(ids.astype(np.int32)),
                        torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
                        to_device(x_bits), y, ws, flags)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16), ws


def _check(lay, ids, w, x_bits, y_bits):
    y_o = O.grouped_layer(lay.experts, ids, w.astype(np.float64), x_bits, lay.S.group,
                          lay.loras, lay.scale)
    rels = [rel_l2(O.bf16_to_f64(y_bits[j]), y_o[j]) for j in range(ids.shape[0])]
    assert max(rels) <= REL_L2_MAX, (max(rels), int(np.argmax(rels)))
    return max(rels)


@pytest.mark.parametrize("T", [1, 3, 8, 17, 64])
def test_grouped_tiny(torch_cuda, T):
    S = G.TINY
    lay = _layer(S)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=10 + T)
    x = G.hidden(S, 20 + T, n=T)
    ys = {}
    for flags in FLAG_SETS:
        y, _ = _call(lay, ids, w, x, flags)
        ys[flags] = y
        worst = _check(lay, ids, w, x, y)
        print(f"[grouped] tiny T={T} flags={flags:#x}: worst rel-L2 {worst:.3e}")
    _paths_ran(ys, ids, np.bincount(ids.ravel(), minlength=S.n_experts))


@pytest.mark.parametrize("T", [1, 4, 8, 16, 32, 64])
def test_grouped_qwen3moe_k8(torch_cuda, T):
    S = G.QWEN3_MOE.with_k(8)
    lay = _layer(S)
    ids, w = G.grouped_routing(S.n_experts, 8, T, seed=T)
    x = G.hidden(S, 100 + T, n=T)
    counts = np.bincount(ids.ravel(), minlength=S.n_experts)
    ys = {}
    for flags in FLAG_SETS:
        y, _ = _call(lay, ids, w, x, flags)
        ys[flags] = y
        worst = _check(lay, ids, w, x, y)
        print(f"[grouped] qwen3moe K=8 T={T} flags={flags:#x}: {np.count_nonzero(counts)} experts, "
              f"max {counts.max()} tokens/expert, {int((counts >= 16).sum())} on MFMA; "
              f"worst rel-L2 {worst:.3e}")
    _paths_ran(ys, ids, counts)


def _paths_ran(ys, ids, counts):
    """Tokens routed only to GEMV experts are bit-identical between the two
    calls; a token that uses an MFMA expert shows the MFMA path's rounding
    (at least one must differ when any expert has >= 16 tokens)."""
    big = set(np.nonzero(counts >= 16)[0].tolist())
    differs = [not np.array_equal(ys[GEMV][j], ys[MFMA16][j]) for j in range(ids.shape[0])]
    for j in range(ids.shape[0]):
        if not big.intersection(ids[j].tolist()):
            assert not differs[j], j
    if big:
        assert any(differs)


def test_grouped_deterministic_and_workspace_reuse(torch_cuda):
    S = G.QWEN3_MOE.with_k(8)
    lay = _layer(S)
    ids, w = G.grouped_routing(S.n_experts, 8, 32, seed=5)
    x = G.hidden(S, 7, n=32)
    y1, ws = _call(lay, ids, w, x)
    y2, ws = _call(lay, ids, w, x, ws=ws)
    assert np.array_equal(y1, y2)
    # a smaller call on the same workspace
    y3, ws = _call(lay, ids[:4], w[:4], x[:4], ws=ws)
    _check(lay, ids[:4], w[:4], x[:4], y3)
    # on the GEMV and tile paths each token alone equals the grouped call's
    # row for it: a token's arithmetic does not depend on the other tokens of
    # its tile or slice, and the fixed-point sums are exact
    for flags in (TILES, GEMV):
        y5, ws = _call(lay, ids, w, x, flags=flags, ws=ws)
        y4, ws = _call(lay, ids[2:3], w[2:3], x[2:3], flags=flags, ws=ws)
        assert np.array_equal(y4[0], y5[2]), flags


def test_grouped_empty_and_bad_ids(torch_cuda):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    S = G.TINY
    lay = _layer(S)
    ws = E.new_grouped_workspace(lay.sh)
    y = torch.zeros((1, S.d_model), dtype=torch.int16, device="cuda")
    E.edge0_moe_grouped(lay.sh, lay.pool.pool, lay.table, 0, None, None, None, None, ws)
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_grouped(lay.sh, lay.pool.pool, lay.table, 65, None, None, None, None, ws)
    ids = np.array([[0, 1, 99, 3]], np.int32)
    w = np.full((1, 4), 0.25, np.float32)
    x = G.hidden(S, 1, n=1)
    y, ws = _call(lay, ids, w, x, ws=ws)
    assert E.edge0_workspace_error(ws) == E.EDGE0_ERANGE
    # the valid pairs still contribute: equals the call with the bad pair
    # replaced by an unused expert of weight 0
    ids_ok = ids.copy()
    ids_ok[0, 2] = 7
    w_ok = w.copy()
    w_ok[0, 2] = 0.0
    y_ok, ws = _call(lay, ids_ok, w_ok, x, ws=ws)
    assert E.edge0_workspace_error(ws) == E.EDGE0_OK
    assert np.array_equal(y, y_ok)


def test_grouped_repeated_ids(torch_cuda):
    """An id repeated within a token's routing adds that expert's output once
    per repeat (the oracle sums the K terms; the device evaluates the expert
    once with the repeats' weights added); here expert 2 is chosen 3 times by
    each of 9 tokens."""
    S = G.TINY
    lay = _layer(S)
    T = 9
    ids = np.tile(np.array([2, 5, 2, 2], np.int32)[:S.top_k], (T, 1))
    rng = np.random.default_rng(4)
    w = rng.uniform(0.05, 0.5, size=(T, S.top_k)).astype(np.float32)
    x = G.hidden(S, 33, n=T)
    for flags in FLAG_SETS:
        y, _ = _call(lay, ids, w, x, flags)
        worst = _check(lay, ids, w, x, y)
        print(f"[grouped] tiny repeated ids flags={flags:#x}: worst rel-L2 {worst:.3e}")


@pytest.mark.parametrize("name,T", [("tiny", 17), ("qwen3moe_k8", 8)])
def test_grouped_without_lora(torch_cuda, name, T):
    """lora_rank 0: no adapter terms on any path (tiles and GEMV)."""
    S = G.TINY if name == "tiny" else G.QWEN3_MOE.with_k(8)
    lay = DeviceLayer(S, seed=6, layer=1, lora=False)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=40 + T)
    x = G.hidden(S, 60 + T, n=T)
    for flags in FLAG_SETS:
        y, _ = _call(lay, ids, w, x, flags)
        worst = _check(lay, ids, w, x, y)
        print(f"[grouped] {name} no LoRA T={T} flags={flags:#x}: worst rel-L2 {worst:.3e}")


def test_grouped_most_pairs(torch_cuda):
    """64 tokens with K = E = 16 on the tiny shape: 1024 pairs (the most a
    call holds), every expert chosen by every token, so each expert spans
    four 16-token tiles."""
    S = G.TINY.with_k(16)
    lay = DeviceLayer(S, seed=8, layer=2)
    T = 64
    ids, w = G.grouped_routing(S.n_experts, 16, T, seed=77)
    assert all(len(set(row.tolist())) == 16 for row in ids)
    x = G.hidden(S, 90, n=T)
    for flags in FLAG_SETS:
        y, _ = _call(lay, ids, w, x, flags)
        worst = _check(lay, ids, w, x, y)
        print(f"[grouped] tiny K=16 T=64 flags={flags:#x}: worst rel-L2 {worst:.3e}")
