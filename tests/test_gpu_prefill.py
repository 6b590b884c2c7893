"""GPU parity of the whole-layer prefill call (edge0_moe_prefill) against
the oracle's token-by-token definition y_j = sum_k w_jk FFN_{e_jk}(x_j)
([Edge0] §3.1 "Executor paths" whole-layer, "Math contract"): every token
at the tiny shape and at 100 Qwen3-MoE tokens (K = 8, Zipf(1.1) routing),
sampled tokens at 1024 and at 4096 tokens (the most per call), rel-L2 <= 2e-3
per token; bit-identical repeats, a token alone equal to its row of a large
call, a smaller call on the same workspace, ids repeated within a token,
lora_rank 0, the empty call, invalid ids reported, and arguments refused."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, DeviceLayer, check_layer_output, rel_l2

pytestmark = pytest.mark.gpu

_LAYERS = {}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _layer(S, lora=True):
    key = (S.d_model, S.top_k, lora)
    if key not in _LAYERS:
        _LAYERS[key] = DeviceLayer(S, seed=4, layer=1, lora=lora)
    return _LAYERS[key]


def _call(lay, ids, w, x_bits, max_tokens=None, ws=None):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    T = ids.shape[0]
    mt = max_tokens or max(T, 1)
    if ws is None:
        ws = E.new_prefill_workspace(lay.sh, mt)
    y = torch.zeros((T, lay.S.d_model), dtype=torch.int16, device="cuda")
    E.edge0_moe_prefill(lay.sh, lay.pool.pool, lay.table, T, to_device(ids.astype(np.int32)),
                        torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
                        to_device(x_bits), y, ws, mt)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16), ws


def _check(lay, ids, w, x_bits, y_bits, rows):
    """Every listed token's output against the oracle (check_layer_output);
    returns the worst rel-L2 and the worst element error in units of its
    bound."""
    worst, worst_el = 0.0, 0.0
    for j in rows:
        y_o = O.moe_layer(lay.experts, ids[j], w[j].astype(np.float64), x_bits[j], lay.S.group,
                          lay.loras, lay.scale)
        rel, el = check_layer_output(y_bits[j], y_o)
        worst, worst_el = max(worst, rel), max(worst_el, el)
    print(f"[prefill] worst element error {worst_el:.3f} of its bound")
    return worst


@pytest.mark.parametrize("T", [1, 17, 300])
def test_prefill_tiny_every_token(torch_cuda, T):
    S = G.TINY
    lay = _layer(S)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=30 + T)
    x = G.hidden(S, 40 + T, n=T)
    y, _ = _call(lay, ids, w, x)
    worst = _check(lay, ids, w, x, y, range(T))
    print(f"[prefill] tiny T={T}: worst rel-L2 {worst:.3e}")


@pytest.mark.parametrize("T,n_check", [(100, 100), (1024, 48), (4096, 24)])
def test_prefill_qwen3moe_k8(torch_cuda, T, n_check):
    S = G.QWEN3_MOE.with_k(8)
    lay = _layer(S)
    ids, w = G.grouped_routing(S.n_experts, 8, T, seed=T + 1)
    x = G.hidden(S, 200 + T, n=T)
    print(f"[prefill] qwen3moe K=8 T={T}", flush=True)
    y, _ = _call(lay, ids, w, x)
    rows = range(T) if n_check >= T else np.random.default_rng(T).choice(T, n_check, replace=False)
    worst = _check(lay, ids, w, x, y, list(rows))
    counts = np.bincount(ids.ravel(), minlength=S.n_experts)
    print(f"[prefill] qwen3moe K=8 T={T}: {np.count_nonzero(counts)} experts, max {counts.max()} "
          f"tokens/expert; worst rel-L2 {worst:.3e} over {len(list(rows))} tokens")


def test_prefill_deterministic_token_alone_and_reuse(torch_cuda):
    """Pairs take their place in an expert's run in arrival order; a pair's
    result must not depend on it: repeats are bit-identical, and a token
    alone equals its row of the large call."""
    S = G.QWEN3_MOE.with_k(8)
    lay = _layer(S)
    T = 512
    ids, w = G.grouped_routing(S.n_experts, 8, T, seed=77)
    x = G.hidden(S, 78, n=T)
    y1, ws = _call(lay, ids, w, x, max_tokens=T)
    y2, ws = _call(lay, ids, w, x, max_tokens=T, ws=ws)
    assert np.array_equal(y1, y2)
    for j in (0, 5, 300, 511):
        yj, ws = _call(lay, ids[j:j + 1], w[j:j + 1], x[j:j + 1], max_tokens=T, ws=ws)
        assert np.array_equal(yj[0], y1[j]), j
    # a smaller call on the same workspace
    y3, ws = _call(lay, ids[:40], w[:40], x[:40], max_tokens=T, ws=ws)
    _check(lay, ids[:40], w[:40], x[:40], y3, range(40))


def test_prefill_repeated_ids_and_no_lora(torch_cuda):
    S = G.TINY
    lay = _layer(S)
    T = 64
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=9)
    ids = ids.copy()
    ids[3, 1] = ids[3, 0]            # one repeat
    ids[10, :] = ids[10, 0]          # all K the same expert
    y, _ = _call(lay, ids, w, G.hidden(S, 9, n=T))
    _check(lay, ids, w, G.hidden(S, 9, n=T), y, range(T))
    for S2 in (G.TINY, G.QWEN3_MOE.with_k(8)):
        lay0 = _layer(S2, lora=False)
        T2 = 48
        ids2, w2 = G.grouped_routing(S2.n_experts, S2.top_k, T2, seed=11)
        x2 = G.hidden(S2, 12, n=T2)
        y2, _ = _call(lay0, ids2, w2, x2)
        _check(lay0, ids2, w2, x2, y2, range(T2))


def test_prefill_empty_bad_ids_and_refusals(torch_cuda):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = G.TINY
    lay = _layer(S)
    ws = E.new_prefill_workspace(lay.sh, 32)
    y = torch.zeros((1, S.d_model), dtype=torch.int16, device="cuda")
    E.edge0_moe_prefill(lay.sh, lay.pool.pool, lay.table, 0, None, None, None, None, ws, 32)
    # an id out of range: reported, its pair contributes nothing
    ids, w = G.grouped_routing(S.n_experts, S.top_k, 8, seed=3)
    bad = ids.copy()
    bad[2, 1] = S.n_experts + 5
    x = G.hidden(S, 4, n=8)
    yb, ws = _call(lay, bad, w, x, max_tokens=32, ws=ws)
    assert E.edge0_workspace_error(ws) == E.EDGE0_ERANGE
    keep = [0, 2, 3]
    y_o = O.moe_layer(lay.experts, bad[2][keep], w[2][keep].astype(np.float64), x[2], S.group,
                      lay.loras, lay.scale)
    check_layer_output(yb[2], y_o)
    assert E.edge0_workspace_error(ws) == 0
    # refused: more tokens than the workspace was sized for, or than 4096
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_prefill(lay.sh, lay.pool.pool, lay.table, 33, to_device(ids.astype(np.int32)),
                            torch.zeros(33 * S.top_k, device="cuda"), to_device(x), y, ws, 32)
    assert E.lib.edge0_prefill_workspace_bytes(E.C.byref(lay.sh), 4097) == 0
    assert E.lib.edge0_prefill_workspace_bytes(E.C.byref(lay.sh), 0) == 0
