"""GPU parity of the single-layer entry points against the CPU oracle, on the
tiny layer (16 experts) and the Qwen3-MoE-shaped layer (128 experts, K = 4
and 8), called through the C ABI."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, DeviceLayer, check_routing, rel_l2

pytestmark = pytest.mark.gpu

SHAPES = {"tiny": G.TINY, "qwen3moe_k4": G.QWEN3_MOE, "qwen3moe_k8": G.QWEN3_MOE.with_k(8)}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


_layers = {}


def layer(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _layers:
        _layers[key] = DeviceLayer(SHAPES[name], **kw)
    return _layers[key]


def _x(S, i):
    from int4_expert_streaming_amd.weights import to_device
    x = G.hidden(S, 0, i)
    return x, to_device(x)


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", list(SHAPES))
def test_router_parity(torch_cuda, name):
    L = layer(name)
    S = L.S
    print(f"[router] {name}", flush=True)
    stats = []
    for i in range(8):
        x, xd = _x(S, i)
        ids, w = L.new_routing()
        logits = torch_cuda.zeros(S.n_experts, dtype=torch_cuda.float32, device="cuda")
        L.E.edge0_router(L.sh, L.wr_d, xd, logits, ids, w, L.ws)
        lo = O.router_logits(L.wr, x)
        lg = logits.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lg - lo)) <= 1e-5 * max(1.0, np.max(np.abs(lo)))
        stats.append(check_routing(ids.cpu().numpy(), w.cpu().numpy(), lo, S.top_k))
    assert L.E.edge0_workspace_error(L.ws) == 0
    assert stats.count("exact") >= 6, stats


@pytest.mark.parametrize("name", list(SHAPES))
def test_prerouter_parity(torch_cuda, name):
    L = layer(name)
    S = L.S
    print(f"[prerouter] {name}", flush=True)
    rng = np.random.default_rng(5)
    stats = []
    for i in range(6):
        x, xd = _x(S, 100 + i)
        now = rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        prev = None if i == 0 else rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        now_d = torch_cuda.tensor(now, device="cuda")
        prev_d = None if prev is None else torch_cuda.tensor(prev, device="cuda")
        ids, w = L.new_routing()
        logits = torch_cuda.zeros(S.n_experts, dtype=torch_cuda.float32, device="cuda")
        L.E.edge0_prerouter(L.sh, L.E.make_head(L.head_d), xd, now_d, prev_d, logits, ids, w, L.ws)
        lo = O.prerouter_logits(L.head, x, now, prev, S.n_experts)
        lg = logits.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lg - lo)) <= 2e-5 * max(1.0, np.max(np.abs(lo))), np.max(np.abs(lg - lo))
        stats.append(check_routing(ids.cpu().numpy(), w.cpu().numpy(), lo, S.top_k))
    assert L.E.edge0_workspace_error(L.ws) == 0
    assert stats.count("exact") >= 4, stats


@pytest.mark.parametrize("name", list(SHAPES))
def test_moe_layer_parity(torch_cuda, name):
    L = layer(name)
    S = L.S
    rng = np.random.default_rng(11)
    worst = 0.0
    for i in range(4):
        print(f"[moe] {name} case {i}", flush=True)
        x, xd = _x(S, 200 + i)
        ids = rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
        w = rng.uniform(0.1, 1.0, S.top_k).astype(np.float32)
        w /= w.sum()
        y = torch_cuda.zeros(S.d_model, dtype=torch_cuda.int16, device="cuda")
        L.E.edge0_moe_layer(L.sh, L.pool.pool, L.table, torch_cuda.tensor(ids, device="cuda"),
                            torch_cuda.tensor(w, device="cuda"), xd, y, L.ws)
        yo = L.oracle_y(ids, w.astype(np.float64), x)
        rel = rel_l2(O.bf16_to_f64(_bits(y)), yo)
        worst = max(worst, rel)
        assert rel <= REL_L2_MAX, rel
    assert L.E.edge0_workspace_error(L.ws) == 0
    print(f"[moe] {name} worst rel-L2 {worst:.3e}")


def test_moe_layer_permuted_slots(torch_cuda):
    """The slot table maps ids to slots on the device (take): a permuted pool
    gives the same output as the identity pool."""
    S = G.TINY
    perm = np.random.default_rng(3).permutation(S.n_experts)
    A = layer("tiny")
    B = layer("tiny", slot_perm=tuple(perm.tolist()))
    x, xd = _x(S, 7)
    ids = torch_cuda.tensor([3, 11, 0, 15], dtype=torch_cuda.int32, device="cuda")
    w = torch_cuda.tensor([0.4, 0.3, 0.2, 0.1], dtype=torch_cuda.float32, device="cuda")
    ya = torch_cuda.zeros(S.d_model, dtype=torch_cuda.int16, device="cuda")
    yb = torch_cuda.zeros_like(ya)
    A.E.edge0_moe_layer(A.sh, A.pool.pool, A.table, ids, w, xd, ya, A.ws)
    B.E.edge0_moe_layer(B.sh, B.pool.pool, B.table, ids, w, xd, yb, B.ws)
    assert torch_cuda.equal(ya, yb)


@pytest.mark.parametrize("name", ["tiny", "qwen3moe_k4"])
def test_moe_layer_deterministic_and_lora_zero(torch_cuda, name):
    """Two runs are bit-identical; B = 0 adapters give exactly the no-adapter
    output."""
    S = SHAPES[name]
    L = layer(name)
    x, xd = _x(S, 9)
    ids = torch_cuda.tensor(list(range(S.top_k)), dtype=torch_cuda.int32, device="cuda")
    w = torch_cuda.full((S.top_k,), 1.0 / S.top_k, dtype=torch_cuda.float32, device="cuda")
    outs = []
    for _ in range(2):
        y = torch_cuda.zeros(S.d_model, dtype=torch_cuda.int16, device="cuda")
        L.E.edge0_moe_layer(L.sh, L.pool.pool, L.table, ids, w, xd, y, L.ws)
        outs.append(y)
    assert torch_cuda.equal(outs[0], outs[1])
    # zero every B factor in place (the pool holds the adapters) and compare
    # with a rank-0 pool of the same experts
    N = layer(name, lora=False)
    lay = L.pool.layout
    Z = DeviceLayer(S)
    for s in range(S.n_experts):
        b = Z.pool.bundle_bytes(s)
        for key, n in (("b_gate", S.d_inter), ("b_up", S.d_inter), ("b_down", S.d_model)):
            off = getattr(lay, key)
            b[off:off + n * S.lora_rank * 2].zero_()
    yz = torch_cuda.zeros(S.d_model, dtype=torch_cuda.int16, device="cuda")
    yn = torch_cuda.zeros_like(yz)
    Z.E.edge0_moe_layer(Z.sh, Z.pool.pool, Z.table, ids, w, xd, yz, Z.ws)
    N.E.edge0_moe_layer(N.sh, N.pool.pool, N.table, ids, w, xd, yn, N.ws)
    assert torch_cuda.equal(yz, yn)
    assert not torch_cuda.equal(yz, outs[0])


@pytest.mark.parametrize("name", ["tiny", "qwen3moe_k8"])
def test_bad_ids_are_reported_not_dereferenced(torch_cuda, name):
    """An id outside [0, E) or a slot of -1 is skipped on the device and
    reported through the workspace error word (the narrow-row launches on the
    tiny shape, the fused layer kernel and its down launch on the wide one)."""
    S = SHAPES[name]
    K = S.top_k
    L = layer(name)
    x, xd = _x(S, 1)
    w = torch_cuda.full((K,), 1.0 / K, dtype=torch_cuda.float32, device="cuda")
    y = torch_cuda.zeros(S.d_model, dtype=torch_cuda.int16, device="cuda")
    good = [5] + [e for e in range(1, K + 1) if e != 5][:K - 1]
    bad = list(good)
    bad[2] = S.n_experts + 3
    L.E.edge0_moe_layer(L.sh, L.pool.pool, L.table,
                        torch_cuda.tensor(bad, dtype=torch_cuda.int32, device="cuda"), w, xd, y,
                        L.ws)
    assert L.E.edge0_workspace_error(L.ws) == L.E.EDGE0_ERANGE
    table = L.table.clone()
    table[5] = -1
    ids = torch_cuda.tensor(good, dtype=torch_cuda.int32, device="cuda")
    L.E.edge0_moe_layer(L.sh, L.pool.pool, table, ids, w, xd, y, L.ws)
    assert L.E.edge0_workspace_error(L.ws) == L.E.EDGE0_ERANGE
    # the remaining experts still combine: compare with the oracle over the others
    yo = L.oracle_y(good[1:], [1.0 / K] * (K - 1), x)
    assert rel_l2(O.bf16_to_f64(_bits(y)), yo) <= REL_L2_MAX
    # and the next call on the same workspace is clean
    L.E.edge0_moe_layer(L.sh, L.pool.pool, L.table, ids, w, xd, y, L.ws)
    assert L.E.edge0_workspace_error(L.ws) == 0


@pytest.mark.parametrize("name", ["tiny", "qwen3moe_k8"])
def test_router_exact_ties_rank_by_index(torch_cuda, name):
    """Experts whose router rows are identical get identical logits; the
    committed top-K must rank that tie by ascending expert index, as the
    oracle's (value descending, index ascending) order does.  Four copies of
    the row that scores highest make the top four a pure tie."""
    from int4_expert_streaming_amd.weights import to_device
    L = layer(name)
    S = L.S
    x, xd = _x(S, 3)
    lo = O.router_logits(L.wr, x)
    top = int(np.argmax(lo))
    copies = sorted({top, (top + 1) % S.n_experts, (top + 5) % S.n_experts, 3 % S.n_experts})
    wr = L.wr.copy()
    for e in copies:
        wr[e] = L.wr[top]
    wr_d = to_device(wr)
    ids, w = L.new_routing()
    logits = torch_cuda.zeros(S.n_experts, dtype=torch_cuda.float32, device="cuda")
    L.E.edge0_router(L.sh, wr_d, xd, logits, ids, w, L.ws)
    lg = logits.cpu().numpy()
    assert len(set(lg[copies].tolist())) == 1  # the copies' logits are bit-identical
    lo2 = O.router_logits(wr, x)
    ids_o, _ = O.softmax_topk(lo2, S.top_k)
    got = ids.cpu().numpy()
    assert list(ids_o[:len(copies)]) == copies  # the oracle's order
    assert list(got[:len(copies)]) == copies, (got, copies)
    # the rest of the set and the weights as in the other router checks
    check_routing(got, w.cpu().numpy(), lo2, S.top_k)
    assert L.E.edge0_workspace_error(L.ws) == 0
