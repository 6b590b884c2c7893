"""The layer with its LoRA given apart from the bundles (edge0_moe_layer_lora,
[Edge0] §3.3: adapters ship beside the base weights): per-expert adapters in
blocks of their own over a pool of LoRA-free bundles, bit-identical to
edge0_moe_layer with the same adapters inside the bundles; one adapter
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
