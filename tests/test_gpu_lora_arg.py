"""The layer, grouped and prefill calls with their LoRA given apart from the
bundles (edge0_moe_layer_lora, edge0_moe_grouped_lora, edge0_moe_prefill_lora;
[Edge0] §3.3: adapters ship beside the base weights): per-expert adapters in
blocks of their own over a pool of LoRA-free bundles, bit-identical to the
bundled calls with the same adapters inside the bundles (the grouped call on
its GEMV and its MFMA-tile paths, prefill at several sizes); one adapter
shared by every expert (stride 0) against the oracle; arguments refused."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import DeviceLayer, check_layer_output

pytestmark = pytest.mark.gpu

FACTORS = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _adapters(loras, experts):
    """Device block per expert [a_gate|b_gate|a_up|b_up|a_down|b_down] and the
    Lora struct pointing at expert 0's factors, stride one block."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    blocks = [np.concatenate([loras[e][f].ravel() for f in FACTORS]) for e in experts]
    stride = blocks[0].size
    buf = torch.from_numpy(np.ascontiguousarray(np.stack(blocks)).view(np.int16)).cuda()
    offs = np.cumsum([0] + [loras[experts[0]][f].size for f in FACTORS])
    base = buf.data_ptr()
    lo = E.Lora(*[base + 2 * int(offs[i]) for i in range(6)], stride)
    return lo, buf


@pytest.mark.parametrize("name,S", [("tiny", G.TINY), ("qwen3moe_k4", G.QWEN3_MOE),
                                    ("qwen3moe_k8", G.QWEN3_MOE.with_k(8))])
def test_separate_adapters_equal_bundled(torch_cuda, name, S):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import SlotPoolBuffer, to_device
    lay = DeviceLayer(S, seed=9, layer=4)
    En = S.n_experts
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    pool0 = SlotPoolBuffer(sh0, En)
    for e in range(En):
        pool0.load(e, lay.experts[e])
    lo, keep = _adapters(lay.loras, list(range(En)))
    ws = E.new_workspace(lay.sh)
    rng = np.random.default_rng(3)
    for i in range(6):
        x = to_device(G.hidden(S, 60 + i))
        ids = torch.from_numpy(rng.choice(En, S.top_k, replace=False).astype(np.int32)).cuda()
        wv = rng.uniform(0.1, 1.0, S.top_k)
        w = torch.from_numpy((wv / wv.sum()).astype(np.float32)).cuda()
        y_b = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
        y_s = torch.zeros_like(y_b)
        E.edge0_moe_layer(lay.sh, lay.pool.pool, lay.table, ids, w, x, y_b, ws)
        E.edge0_moe_layer_lora(lay.sh, pool0.pool, lo, lay.table, ids, w, x, y_s, ws)
        torch.cuda.synchronize()
        assert torch.equal(y_b, y_s), (name, i)
    assert E.edge0_workspace_error(ws) == 0
    print(f"[lora-arg] {name}: separate adapters bit-identical to bundled ones")


def test_shared_adapter_against_oracle(torch_cuda):
    """expert_stride 0: every expert uses one adapter."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import SlotPoolBuffer, to_device
    S = G.QWEN3_MOE
    lay = DeviceLayer(S, seed=10, layer=0)
    En = S.n_experts
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    pool0 = SlotPoolBuffer(sh0, En)
    for e in range(En):
        pool0.load(e, lay.experts[e])
    shared = G.lora_tensors(S, 10, 0, 999)
    lo, keep = _adapters({0: shared}, [0])
    lo.expert_stride = 0
    ws = E.new_workspace(lay.sh)
    rng = np.random.default_rng(4)
    for i in range(4):
        xb = G.hidden(S, 80 + i)
        ids = rng.choice(En, S.top_k, replace=False).astype(np.int32)
        w = np.full(S.top_k, 1.0 / S.top_k, np.float32)
        y = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
        E.edge0_moe_layer_lora(lay.sh, pool0.pool, lo, lay.table, torch.from_numpy(ids).cuda(),
                               torch.from_numpy(w).cuda(), to_device(xb), y, ws)
        torch.cuda.synchronize()
        y_o = O.moe_layer(lay.experts, ids, w.astype(np.float64), xb, S.group,
                          {e: shared for e in range(En)}, lay.scale)
        check_layer_output(y.cpu().numpy().view(np.uint16), y_o)


def test_lora_argument_refusals(torch_cuda):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = G.TINY
    lay = DeviceLayer(S, seed=11, layer=0)
    ws = E.new_workspace(lay.sh)
    x = to_device(G.hidden(S, 1))
    y = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    ids = torch.arange(S.top_k, dtype=torch.int32, device="cuda")
    w = torch.full((S.top_k,), 0.25, dtype=torch.float32, device="cuda")
    with pytest.raises(E.Edge0Error):  # rank 8 without adapters
        E.edge0_moe_layer_lora(lay.sh, lay.pool.pool, None, lay.table, ids, w, x, y, ws)
    lo, keep = _adapters(lay.loras, list(range(S.n_experts)))
    lo.expert_stride = -1
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_layer_lora(lay.sh, lay.pool.pool, lo, lay.table, ids, w, x, y, ws)
    # rank 0: no adapters needed, the base layer alone
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    E.edge0_moe_layer_lora(sh0, lay.pool.pool, None, lay.table, ids, w, x, y, ws)
    torch.cuda.synchronize()
    y_o = O.moe_layer(lay.experts, np.arange(S.top_k), np.full(S.top_k, 0.25), G.hidden(S, 1), S.group)
    check_layer_output(y.cpu().numpy().view(np.uint16), y_o)


def _pool0(E, S, lay):
    """A pool of LoRA-free bundles holding the layer's int4 experts."""
    from int4_expert_streaming_amd.weights import SlotPoolBuffer
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    pool0 = SlotPoolBuffer(sh0, S.n_experts)
    for e in range(S.n_experts):
        pool0.load(e, lay.experts[e])
    return pool0


@pytest.mark.parametrize("name,S,T,flags", [
    ("tiny", G.TINY, 5, 0), ("tiny", G.TINY, 20, 1),
    ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 1, 0), ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 2, 0),
    ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 32, 0), ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 32, 1)])
def test_grouped_separate_adapters_equal_bundled(torch_cuda, name, S, T, flags):
    """flags 1: every expert on the GEMVs; 0: the MFMA tiles from 3 tokens."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    lay = DeviceLayer(S, seed=12, layer=2)
    pool0 = _pool0(E, S, lay)
    lo, keep = _adapters(lay.loras, list(range(S.n_experts)))
    ws = E.new_grouped_workspace(lay.sh)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=70 + T)
    x = to_device(G.hidden(S, 90 + T, n=T))
    ids_d = to_device(ids.astype(np.int32))
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    y_b = torch.zeros((T, S.d_model), dtype=torch.int16, device="cuda")
    y_s = torch.zeros_like(y_b)
    E.edge0_moe_grouped(lay.sh, lay.pool.pool, lay.table, T, ids_d, w_d, x, y_b, ws, flags)
    E.edge0_moe_grouped_lora(lay.sh, pool0.pool, lo, lay.table, T, ids_d, w_d, x, y_s, ws, flags)
    torch.cuda.synchronize()
    assert torch.equal(y_b, y_s), (name, T, flags)
    assert E.edge0_workspace_error(ws) == 0


@pytest.mark.parametrize("name,S,T", [("tiny", G.TINY, 17), ("tiny", G.TINY, 300),
                                      ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 100),
                                      ("qwen3moe_k8", G.QWEN3_MOE.with_k(8), 1024)])
def test_prefill_separate_adapters_equal_bundled(torch_cuda, name, S, T):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    lay = DeviceLayer(S, seed=13, layer=3)
    pool0 = _pool0(E, S, lay)
    lo, keep = _adapters(lay.loras, list(range(S.n_experts)))
    ws = E.new_prefill_workspace(lay.sh, T)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=110 + T)
    x = to_device(G.hidden(S, 130 + T, n=T))
    ids_d = to_device(ids.astype(np.int32))
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    y_b = torch.zeros((T, S.d_model), dtype=torch.int16, device="cuda")
    y_s = torch.zeros_like(y_b)
    E.edge0_moe_prefill(lay.sh, lay.pool.pool, lay.table, T, ids_d, w_d, x, y_b, ws, T)
    E.edge0_moe_prefill_lora(lay.sh, pool0.pool, lo, lay.table, T, ids_d, w_d, x, y_s, ws, T)
    torch.cuda.synchronize()
    assert torch.equal(y_b, y_s), (name, T)
    assert E.edge0_workspace_error(ws) == 0


def test_prefill_shared_adapter_against_oracle(torch_cuda):
    """expert_stride 0 on the prefill call: every expert uses one adapter."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE.with_k(8)
    lay = DeviceLayer(S, seed=14, layer=0)
    pool0 = _pool0(E, S, lay)
    shared = G.lora_tensors(S, 14, 0, 999)
    lo, keep = _adapters({0: shared}, [0])
    lo.expert_stride = 0
    T = 64
    ws = E.new_prefill_workspace(lay.sh, T)
    ids, w = G.grouped_routing(S.n_experts, S.top_k, T, seed=150)
    xb = G.hidden(S, 151, n=T)
    y = torch.zeros((T, S.d_model), dtype=torch.int16, device="cuda")
    E.edge0_moe_prefill_lora(lay.sh, pool0.pool, lo, lay.table, T, to_device(ids.astype(np.int32)),
                             torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
                             to_device(xb), y, ws, T)
    torch.cuda.synchronize()
    yb = y.cpu().numpy().view(np.uint16)
    for j in range(0, T, 7):
        y_o = O.moe_layer(lay.experts, ids[j], w[j].astype(np.float64), xb[j], S.group,
                          {e: shared for e in range(S.n_experts)}, lay.scale)
        check_layer_output(yb[j], y_o)


def test_grouped_prefill_lora_refusals(torch_cuda):
    import torch
    from int4_expert_streaming_amd import edge0 as E
    S = G.TINY
    lay = DeviceLayer(S, seed=15, layer=0)
    wsg = E.new_grouped_workspace(lay.sh)
    wsp = E.new_prefill_workspace(lay.sh, 4)
    with pytest.raises(E.Edge0Error):  # rank 8 without adapters
        E.edge0_moe_grouped_lora(lay.sh, lay.pool.pool, None, lay.table, 0, None, None, None,
                                 None, wsg)
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_prefill_lora(lay.sh, lay.pool.pool, None, lay.table, 0, None, None, None,
                                 None, wsp, 4)
    lo, keep = _adapters(lay.loras, list(range(S.n_experts)))
    lo.expert_stride = -1
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_grouped_lora(lay.sh, lay.pool.pool, lo, lay.table, 0, None, None, None,
                                 None, wsg)
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_prefill_lora(lay.sh, lay.pool.pool, lo, lay.table, 0, None, None, None,
                                 None, wsp, 4)
    # a pool too small for the bundled call but right for LoRA-free bundles
    pool0 = _pool0(E, S, lay)
    with pytest.raises(E.Edge0Error):
        E.edge0_moe_grouped(lay.sh, pool0.pool, lay.table, 0, None, None, None, None, wsg)
    lo.expert_stride = 0
    E.edge0_moe_grouped_lora(lay.sh, pool0.pool, lo, lay.table, 0, None, None, None, None, wsg)
    torch.cuda.synchronize()
