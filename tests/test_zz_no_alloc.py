"""The no-allocation single-layer entry point (edge0_moe_layer_noalloc)
against edge0_moe_layer on a caller workspace: the same kernels on the
library's static per-GPU scratch, so outputs must be bit-identical.  Two
calls in a row, the second on a smaller shape (the tiny layer after the
Qwen3-MoE-shaped one), then the first shape again on the reused scratch;
error reporting through error_out; a shape whose workspace exceeds the
static array is refused before anything is enqueued."""
import numpy as np
import pytest

from synth import gen as G
from tests.layer_setup import DeviceLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(torch, L, ids, w, x_bits):
    from int4_expert_streaming_amd.weights import to_device
    E = L.E
    S = L.S
    idt = torch.tensor(ids, dtype=torch.int32, device="cuda")
    wt = torch.tensor(w, dtype=torch.float32, device="cuda")
    xd = to_device(x_bits)
    y_ref = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    y = torch.full((S.d_model,), 0x7FC0, dtype=torch.int16, device="cuda")
    err = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    E.edge0_moe_layer(L.sh, L.pool.pool, L.table, idt, wt, xd, y_ref, L.ws)
    ref_err = E.edge0_workspace_error(L.ws)
    E.edge0_moe_layer_noalloc(L.sh, L.pool.pool, L.table, idt, wt, xd, y, err)
    torch.cuda.synchronize()
    return (y_ref.cpu().numpy().view(np.uint16), y.cpu().numpy().view(np.uint16), ref_err,
            int(err.cpu()[0]))


def test_noalloc_matches_workspace_call(torch_cuda):
    from int4_expert_streaming_amd import edge0 as E
    torch = torch_cuda
    big = DeviceLayer(G.QWEN3_MOE.with_k(8), seed=1, layer=2)
    small = DeviceLayer(G.TINY, seed=1, layer=3)
    rng = np.random.default_rng(2)
    for L, tag in ((big, "qwen3moe K=8"), (small, "tiny"), (big, "qwen3moe K=8 again")):
        S = L.S
        ids = rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        w = rng.uniform(0.1, 1.0, S.top_k).astype(np.float32)
        w /= w.sum()
        y_ref, y, ref_err, err = _both(torch, L, ids, w, G.hidden(S, 5, int(rng.integers(100))))
        assert ref_err == E.EDGE0_OK and err == E.EDGE0_OK, (ref_err, err)
        assert np.array_equal(y, y_ref), tag
        print(f"[noalloc] {tag}: bit-identical to the workspace call")
    # an out-of-range id: reported through error_out, and the next call is clean
    S = small.S
    ids = np.array([0, 1, 99, 3], np.int32)
    w = np.full(4, 0.25, np.float32)
    y_ref, y, ref_err, err = _both(torch, small, ids, w, G.hidden(S, 6))
    assert ref_err == E.EDGE0_ERANGE and err == E.EDGE0_ERANGE
    assert np.array_equal(y, y_ref)
    ids = np.array([0, 1, 2, 3], np.int32)
    y_ref, y, ref_err, err = _both(torch, small, ids, w, G.hidden(S, 7))
    assert ref_err == E.EDGE0_OK and err == E.EDGE0_OK
    assert np.array_equal(y, y_ref)
    # the same on the wide shape (fused layer kernel and its down launch)
    S = big.S
    ids = np.array([0, 1, 2, 3, S.n_experts + 7, 5, 6, 9], np.int32)
    w = np.full(S.top_k, 1.0 / S.top_k, np.float32)
    y_ref, y, ref_err, err = _both(torch, big, ids, w, G.hidden(S, 8))
    assert ref_err == E.EDGE0_ERANGE and err == E.EDGE0_ERANGE
    assert np.array_equal(y, y_ref)
    ids[4] = 4
    y_ref, y, ref_err, err = _both(torch, big, ids, w, G.hidden(S, 9))
    assert ref_err == E.EDGE0_OK and err == E.EDGE0_OK
    assert np.array_equal(y, y_ref)


def test_noalloc_refuses_oversized_shape(torch_cuda):
    from int4_expert_streaming_amd import edge0 as E
    torch = torch_cuda
    sh = E.make_shape(G.MoEShape(8192, 64, 4096, 16, 64, 64, 128.0, 0))
    assert E.edge0_workspace_bytes(sh) > E.EDGE0_STATIC_WORKSPACE_BYTES
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    pool = E.SlotPool(dummy.data_ptr(), 1 << 30, 1)
    with pytest.raises(E.Edge0Error) as ei:
        E.edge0_moe_layer_noalloc(sh, pool, dummy, dummy, dummy, dummy, dummy + 1)
    assert ei.value.code == E.EDGE0_ESCRATCH
