"""GPU parity of sigmoid-group routing ([Edge0] App. A "Sigmoid-group (K, G
of n groups, scale s)", §2 "MoE routing") against the oracle, through the C
ABI: the commit alone on seeded logits (with and without a selection bias,
exact ties, saturated scores), and the router and prerouter calls with the
family set in the shape."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import W_REL_MAX, DeviceLayer

pytestmark = pytest.mark.gpu

# (E, n groups, G surviving, K, scale): the 8B tier's n=8, G=4, s=2.5, K=8
# at E=128, and shapes that stress group size, group count and K.
CONFIGS = [(16, 4, 2, 4, 1.0), (128, 8, 4, 8, 2.5), (256, 8, 4, 8, 2.5), (1024, 64, 8, 16, 1.5),
           (64, 1, 1, 6, 1.0), (128, 64, 64, 8, 2.5), (96, 3, 2, 5, 0.7)]
SIGMA_GAP = 1e-6   # commit from identical fp32 logits: only the sigmoid's last ulps differ


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _shape(E_mod, Ex, n, Gs, K, s):
    from types import SimpleNamespace
    base = SimpleNamespace(d_model=256, n_experts=Ex, d_inter=128, top_k=K, group=32, lora_rank=0,
                           lora_alpha=0.0, head_hidden=0)
    return E_mod.make_shape(base, E_mod.EDGE0_ROUTE_SIGMOID_GROUP, n, Gs, s)


def _check(gpu_ids, gpu_w, logits, K, n, Gs, s, bias, gap, exact_only=False):
    """"exact" when ids (in order) and weights match the oracle's; "waived"
    when a group or expert decision has a margin below `gap` (then only the
    properties every valid answer has are checked)."""
    gpu_ids = np.asarray(gpu_ids).tolist()
    gpu_w = np.asarray(gpu_w, dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    ids, w = O.sigmoid_group_topk(logits, K, n, Gs, s, bias)
    if not exact_only and min(O.sigmoid_group_gaps(logits, K, n, Gs, bias)) < gap:
        E = len(logits)
        assert len(set(gpu_ids)) == K and all(0 <= e < E for e in gpu_ids)
        assert len({e // (E // n) for e in gpu_ids}) <= Gs
        want = s * sig[gpu_ids] / (sig[gpu_ids].sum() + 1e-20)
        np.testing.assert_allclose(gpu_w, want, rtol=W_REL_MAX, atol=1e-30)
        return "waived"
    assert sorted(gpu_ids) == sorted(ids.tolist()), (gpu_ids, ids.tolist())
    # within the set, the rank order may differ only between scores closer
    # than `gap` (exact_only: not at all)
    c = sig + (0.0 if bias is None else np.asarray(bias, np.float64))
    for a, b in zip(gpu_ids, ids.tolist()):
        if a != b:
            assert not exact_only and abs(c[a] - c[b]) < gap, (gpu_ids, ids.tolist())
    want = dict(zip(ids.tolist(), w.tolist()))
    np.testing.assert_allclose(gpu_w, [want[e] for e in gpu_ids], rtol=W_REL_MAX, atol=1e-30)
    return "exact"


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "E{}_n{}_G{}_K{}".format(*c[:4]))
def test_commit_parity(torch_cuda, cfg):
    from int4_expert_streaming_amd import edge0 as E
    Ex, n, Gs, K, s = cfg
    print(f"[commit] {cfg}", flush=True)
    sh = _shape(E, Ex, n, Gs, K, s)
    rng = np.random.default_rng(Ex * 131 + n)
    stats = []
    for i in range(24):
        spread = [0.5, 2.0, 8.0][i % 3]
        logits = (rng.normal(0.0, spread, Ex)).astype(np.float32)
        bias = None if i % 4 == 0 else (rng.normal(0.0, [0.05, 0.3, 1.0][i % 3], Ex)).astype(np.float32)
        ld = torch_cuda.tensor(logits, device="cuda")
        bd = None if bias is None else torch_cuda.tensor(bias, device="cuda")
        ids = torch_cuda.zeros(K, dtype=torch_cuda.int32, device="cuda")
        w = torch_cuda.zeros(K, dtype=torch_cuda.float32, device="cuda")
        E.edge0_route_commit(sh, ld, ids, w, route_bias=bd)
        stats.append(_check(ids.cpu().numpy(), w.cpu().numpy(), logits.astype(np.float64), K, n, Gs,
                            s, bias, SIGMA_GAP))
    assert stats.count("exact") >= 20, stats


def test_commit_exact_ties_and_saturation(torch_cuda):
    """Logits from a few values whose sigmoids and pair sums are far apart
    (so every tie, of scores or of group sums, is exact: the lower index and
    the lower group win), and saturated logits
    (sigmoid 0 and 1, weights through the 1e-20 guard)."""
    from int4_expert_streaming_amd import edge0 as E
    rng = np.random.default_rng(3)
    for Ex, n, Gs, K, s in [(16, 4, 2, 4, 1.0), (128, 8, 4, 8, 2.5), (256, 16, 3, 8, 2.5)]:
        sh = _shape(E, Ex, n, Gs, K, s)
        for trial in range(12):
            # every pair sum of these sigmoids differs by > 0.03: the only
            # ties are exact ones
            logits = rng.choice(np.array([-3.0, -1.5, 0.0, 0.7, 2.2], np.float32), Ex)
            if trial % 3 == 2:
                logits = rng.choice(np.array([-1000.0, 0.0, 1000.0], np.float32), Ex)
            if trial == 11:
                logits = np.full(Ex, -1000.0, np.float32)  # every sigma 0: weights 0
            ld = torch_cuda.tensor(logits, device="cuda")
            ids = torch_cuda.zeros(K, dtype=torch_cuda.int32, device="cuda")
            w = torch_cuda.zeros(K, dtype=torch_cuda.float32, device="cuda")
            E.edge0_route_commit(sh, ld, ids, w)
            _check(ids.cpu().numpy(), w.cpu().numpy(), logits.astype(np.float64), K, n, Gs, s, None,
                   0.0, exact_only=True)


@pytest.mark.parametrize("which", ["router", "prerouter"])
def test_router_and_prerouter_sigmoid_group(torch_cuda, which):
    """The Qwen3-MoE-shaped layer (E=128, K=8) with the 8B tier's family
    (n=8, G=4, s=2.5) and a seeded selection bias: logits as the
    softmax-top-K tests, commit against the oracle on the oracle's logits."""
    S = G.QWEN3_MOE.with_k(8)
    L = DeviceLayer(S)
    E = L.E
    sh = E.make_shape(S, E.EDGE0_ROUTE_SIGMOID_GROUP, 8, 4, 2.5)
    print(f"[{which}] sigmoid-group", flush=True)
    rng = np.random.default_rng(11)
    stats = []
    for i in range(8):
        from int4_expert_streaming_amd.weights import to_device
        x = G.hidden(S, 0, 40 + i)
        xd = to_device(x)
        bias = None if i % 2 == 0 else rng.normal(0.0, 0.05, S.n_experts).astype(np.float32)
        bd = None if bias is None else torch_cuda.tensor(bias, device="cuda")
        ids, w = L.new_routing()
        logits = torch_cuda.zeros(S.n_experts, dtype=torch_cuda.float32, device="cuda")
        if which == "router":
            E.edge0_router(sh, L.wr_d, xd, logits, ids, w, L.ws, route_bias=bd)
            lo = O.router_logits(L.wr, x)
        else:
            now = rng.choice(S.n_experts, S.top_k, replace=False).astype(np.int32)
            now_d = torch_cuda.tensor(now, device="cuda")
            E.edge0_prerouter(sh, E.make_head(L.head_d), xd, now_d, None, logits, ids, w, L.ws,
                              route_bias=bd)
            lo = O.prerouter_logits(L.head, x, now, None, S.n_experts)
        lg = logits.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lg - lo)) <= 2e-5 * max(1.0, np.max(np.abs(lo)))
        stats.append(_check(ids.cpu().numpy(), w.cpu().numpy(), lo, S.top_k, 8, 4, 2.5, bias, 1e-4))
    assert E.edge0_workspace_error(L.ws) == 0
    assert stats.count("exact") >= 6, stats
