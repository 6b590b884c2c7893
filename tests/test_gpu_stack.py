"""GPU parity of the decode stack (edge0_stack_*) against the oracle.

Each checked layer is teacher-forced: the oracle takes the GPU's hidden
state entering the layer and, on prediction-routed layers, the GPU's
committed routing, so a near tie waived at one layer cannot cascade.  The
small stack (tiny layer shape, 10 layers) is checked at every layer and also
run free against the oracle; the 40-layer Qwen3-MoE-shaped stack - the one
the benchmark times, in the same launch configuration - is checked at every
layer of several steps, in both execution modes, at K = 4 and K = 8, and with
group biases independent of the scales."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, check_bf16_rounding, check_routing, rel_l2

pytestmark = pytest.mark.gpu


class OracleLayer:
    def __init__(self, gen, L):
        self.gen, self.L = gen, L
        self.router = gen.router(L)
        self.head = gen.head(L)

    def expert(self, e):
        return self.gen.expert(self.L, e)

    def lora(self, e):
        return self.gen.lora(self.L, e)


def _np(t, dt=None):
    a = t.cpu().numpy()
    return a.view(np.uint16) if dt == "bf16" else a


def _snapshot(ds):
    b = ds.stack.buffers()
    return {"x": _np(b["x"], "bf16"), "y": _np(b["y"], "bf16"), "h": _np(b["h"], "bf16"),
            "ids": _np(b["ids"]), "w": _np(b["w"]), "pred_ids": _np(b["pred_ids"]),
            "pred_w": _np(b["pred_w"])}


def check_layer(S, gen, L, t, snap, prev_snap, owners, consumers, report):
    """Teacher-forced comparison of layer L at step t."""
    lay = OracleLayer(gen, L)
    h_in = snap["h"][L]
    # normalised input: the rounding of the exact RMSNorm of the same h, up to
    # near-midpoint cases the fp32 computation may round either way
    check_bf16_rounding(snap["x"][L], O.rmsnorm(O.bf16_to_f64(h_in)))
    x_g = snap["x"][L]
    # routing
    if L in consumers and t > 0:
        assert np.array_equal(snap["ids"][L], prev_snap["pred_ids"][L])
        assert np.array_equal(snap["w"][L], prev_snap["pred_w"][L])
    else:
        report.append(check_routing(snap["ids"][L], snap["w"][L], O.router_logits(lay.router, x_g),
                                    S.top_k))
    # MoE output on the GPU's x and routing
    ids, w = snap["ids"][L], snap["w"][L].astype(np.float64)
    ex = {int(e): lay.expert(int(e)) for e in ids}
    if S.lora_rank > 0:
        lo, scale = {int(e): lay.lora(int(e)) for e in ids}, S.lora_alpha / S.lora_rank
    else:
        lo, scale = None, 0.0
    y_o = O.moe_layer(ex, ids, w, x_g, S.group, lo, scale)
    rel = rel_l2(O.bf16_to_f64(snap["y"][L]), y_o)
    assert rel <= REL_L2_MAX, (L, t, rel)
    # residual: h' = bf16(h + y)
    h_next = O.f64_to_bf16_bits(O.bf16_to_f64(h_in) + O.bf16_to_f64(snap["y"][L]))
    assert np.array_equal(h_next, snap["h"][L + 1]), L
    # head prediction for (L+1, t+1)
    if L in owners:
        prev = None if t == 0 else prev_snap["ids"][L]
        logits = O.prerouter_logits(lay.head, x_g, ids, prev, S.n_experts)
        report.append(check_routing(snap["pred_ids"][L + 1], snap["pred_w"][L + 1], logits,
                                    S.top_k))
    return rel


def _run(ds, S, seed, steps, layers_of, owners, consumers, free_bias=False):
    import torch
    from int4_expert_streaming_amd.weights import to_device
    gen = G.StackGen(S, seed, free_bias=free_bias)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    prev, report, rels = None, [], []
    for t in range(steps):
        print(f"[stack] step {t}", flush=True)
        h0 = G.stack_hidden(S, seed, t)
        ds.step(to_device(h0), h_out, t)
        snap = _snapshot(ds)
        assert np.array_equal(snap["h"][0], h0)
        assert np.array_equal(h_out.cpu().numpy().view(np.uint16), snap["h"][-1])
        for L in layers_of(t):
            rels.append(check_layer(S, gen, L, t, snap, prev, owners, consumers, report))
        prev = snap
    return report, rels


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_small_stack_every_layer(torch_cuda):
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S, seed = G.TINY, 3
    owners, consumers = range(2, 8), range(3, 9)
    ds = DeviceStack(S, G.StackGen(S, seed), 10, (2, 7), (3, 8))
    report, rels = _run(ds, S, seed, 4, lambda t: range(10), owners, consumers)
    assert report.count("exact") >= 0.9 * len(report), report
    print(f"[stack] tiny: worst rel-L2 {max(rels):.3e}, waived {report.count('waived')}")


def test_small_stack_free_running(torch_cuda):
    """Without teacher forcing the oracle stack follows the GPU routing for
    several steps (until a near tie flips an id); report the agreement."""
    import torch
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    S, seed = G.TINY, 4
    owners, consumers = range(2, 8), range(3, 9)
    ds = DeviceStack(S, G.StackGen(S, seed), 10, (2, 7), (3, 8))
    gen = G.StackGen(S, seed)
    layers = [OracleLayer(gen, L) for L in range(10)]
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    committed, prev_ids, agree, total = {}, {}, 0, 0
    for t in range(4):
        h0 = G.stack_hidden(S, seed, t)
        ds.step(to_device(h0), h_out, t)
        snap = _snapshot(ds)
        _, res, committed, prev_ids = O.stack_step(layers, h0, t, committed, prev_ids, S,
                                                   owners, consumers)
        for L in range(10):
            total += 1
            agree += int(np.array_equal(np.sort(res[L]["ids"]), np.sort(snap["ids"][L])))
    print(f"[stack] free-running routing agreement {agree}/{total}")
    assert agree >= 0.9 * total


def _qwen3_stack(S, seed, free_bias=False):
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    return DeviceStack(S, G.StackGen(S, seed, free_bias=free_bias), 40, (6, 37), (7, 38))


QWEN_OWNERS, QWEN_CONSUMERS = range(6, 38), range(7, 39)


@pytest.mark.timeout(900)
def test_qwen3moe_stack_every_layer(torch_cuda):
    """The 40-layer Qwen3-MoE-shaped stack in the configuration the benchmark
    times (graph replay, K = 4), every layer of 3 steps teacher-forced."""
    S, seed = G.QWEN3_MOE, 0
    ds = _qwen3_stack(S, seed)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == 0
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[stack] qwen3moe graphs: worst rel-L2 {max(rels):.3e}, median {np.median(rels):.3e}, "
          f"waived {report.count('waived')}/{len(report)}")
    ds.stack.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["tiny", "qwen3moe"])
def test_head_schedules_agree_bit_for_bit(torch_cuda, which):
    """The folded head schedule (head L's rows beside the down launches of
    layers L and L+1, the default that the checks above run) and the batched
    heads after the last layer give the same bits in every buffer of every
    step, the predictions included; a restart at step 0 reproduces them."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    if which == "tiny":
        S, seed = G.TINY, 5
        ds = DeviceStack(S, G.StackGen(S, seed), 10, (2, 7), (3, 8))
    else:
        S, seed = G.QWEN3_MOE, 21
        ds = _qwen3_stack(S, seed)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    runs = []
    for sched in (E.EDGE0_HEADS_FOLDED, E.EDGE0_HEADS_AFTER_LAYERS, E.EDGE0_HEADS_FOLDED):
        print(f"[stack] {which}: head schedule {sched}", flush=True)
        ds.stack.set_head_schedule(sched)
        snaps = []
        for t in range(4):
            ds.step(to_device(G.stack_hidden(S, seed, t)), h_out, t)
            snaps.append(_snapshot(ds))
        runs.append(snaps)
    for t in range(4):
        for k in runs[0][t]:
            assert np.array_equal(runs[0][t][k], runs[1][t][k]), (which, t, k)
            assert np.array_equal(runs[0][t][k], runs[2][t][k]), (which, t, k)
    assert ds.stack.error() == E.EDGE0_OK


@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["tiny", "qwen3moe"])
def test_stack_separate_adapters_bit_identical(torch_cuda, which):
    """edge0_stack_create_lora over LoRA-free bundles, each layer's adapters
    in a block of their own, gives the bundled stack's bits in every buffer
    of every step; the one-launch modes refuse such a stack."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    if which == "tiny":
        S, seed, n, own, con = G.TINY, 6, 10, (2, 7), (3, 8)
    else:
        S, seed, n, own, con = G.QWEN3_MOE, 22, 40, (6, 37), (7, 38)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    runs = []
    for sep in (False, True):
        print(f"[stack] {which}: adapters apart {sep}", flush=True)
        ds = DeviceStack(S, G.StackGen(S, seed), n, own, con, log=None, separate_lora=sep)
        snaps = []
        for t in range(4):
            ds.step(to_device(G.stack_hidden(S, seed, t)), h_out, t)
            snaps.append(_snapshot(ds))
        assert ds.stack.error() == E.EDGE0_OK
        if sep:
            assert ds.pool.slot_bytes < E.edge0_bundle_layout_of(ds.sh).bytes  # LoRA-free
            with pytest.raises(E.Edge0Error):
                ds.stack.set_mode(E.EDGE0_STACK_PERSISTENT)
        runs.append(snaps)
        del ds
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    for t in range(4):
        for k in runs[0][t]:
            assert np.array_equal(runs[0][t][k], runs[1][t][k]), (which, t, k)


@pytest.mark.timeout(900)
def test_qwen3moe_stack_free_bias_both_modes(torch_cuda):
    """The same stack with group biases drawn independently of the scales
    (b ~ U[-0.16, 0.04]), so a kernel that ignored b or derived it from s
    fails: every layer of 3 steps in the graph mode, then every layer of 3
    steps in the persistent mode (one cooperative launch per step)."""
    from int4_expert_streaming_amd import edge0 as E
    S, seed = G.QWEN3_MOE, 7
    ds = _qwen3_stack(S, seed, free_bias=True)
    for mode in (E.EDGE0_STACK_GRAPHS, E.EDGE0_STACK_PERSISTENT):
        ds.stack.set_mode(mode)
        report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS,
                            free_bias=True)
        assert ds.stack.error() == E.EDGE0_OK
        assert report.count("exact") >= 0.8 * len(report), report
        print(f"[stack] qwen3moe free bias mode {mode}: worst rel-L2 {max(rels):.3e}, "
              f"median {np.median(rels):.3e}, waived {report.count('waived')}/{len(report)}")
    ds.stack.close()


@pytest.mark.timeout(900)
def test_qwen3moe_stack_k8_every_layer(torch_cuda):
    """The 40-layer Qwen3-MoE-shaped stack at K = 8: every layer of 3 steps
    in the graph mode.  (The persistent mode refuses this shape: its 384
    workgroups of 576 threads do not fit its co-residency rule.)"""
    from int4_expert_streaming_amd import edge0 as E
    S, seed = G.QWEN3_MOE.with_k(8), 2
    ds = _qwen3_stack(S, seed)
    with pytest.raises(E.Edge0Error) as ei:
        ds.stack.set_mode(E.EDGE0_STACK_PERSISTENT)
    assert ei.value.code == E.EDGE0_EINVAL
    for mode in (E.EDGE0_STACK_GRAPHS,):
        ds.stack.set_mode(mode)
        report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
        assert ds.stack.error() == E.EDGE0_OK
        assert report.count("exact") >= 0.8 * len(report), report
        print(f"[stack] qwen3moe K=8 mode {mode}: worst rel-L2 {max(rels):.3e}, "
              f"waived {report.count('waived')}/{len(report)}")
    ds.stack.close()


# Router layers hand their logits between the workgroups of one launch; two
# router-layer launches in a row with the same layer-index parity (1 then 5;
# 6 then the next step's 0) must not see each other's logits.
@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_layers", [6, 7])
def test_router_layers_same_parity_in_a_row(torch_cuda, n_layers):
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S, seed = G.MoEShape(2048, 32, 384, 4, 64, 16, 32.0, 64), 13
    owners, consumers = range(1, 4), range(2, 5)
    ds = DeviceStack(S, G.StackGen(S, seed), n_layers, (1, 3), (2, 4), log=None)
    report, rels = _run(ds, S, seed, 3, lambda t: range(n_layers), owners, consumers)
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[stack] router parity n_layers={n_layers}: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


# Wide layers run the fused layer kernel on every layer after step 0; its LoRA
# producers take 2 A rows each for 8 experts at r = 8 (d_model 4096, two
# 2048-wide halves per thread) and 4 A rows each for 8 experts at r = 16.
WIDE_SHAPES = {
    "d4096_k8_r8": G.MoEShape(4096, 16, 256, 8, 64, 8, 16.0, 64),
    "d2048_k8_r16": G.MoEShape(2048, 32, 384, 8, 64, 16, 32.0, 64),
    # no adapters: the down launch finishes the gate/up rows with no LoRA term
    "d2048_k4_r0": G.MoEShape(2048, 32, 384, 4, 64, 0, 0.0, 64),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(WIDE_SHAPES))
def test_wide_stack_every_layer(torch_cuda, name):
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S, seed = WIDE_SHAPES[name], 11
    owners, consumers = range(1, 5), range(2, 6)
    ds = DeviceStack(S, G.StackGen(S, seed), 6, (1, 4), (2, 5))
    report, rels = _run(ds, S, seed, 3, lambda t: range(6), owners, consumers)
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[stack] {name}: worst rel-L2 {max(rels):.3e}, waived {report.count('waived')}")


@pytest.mark.timeout(900)
def test_qwen3moe_stack_persistent_every_layer(torch_cuda):
    """The persistent mode (one cooperative launch for the 40 layers): router
    layers at step 0 and at 0-6 and 39, prediction-routed layers after,
    every layer of 4 steps teacher-forced."""
    from int4_expert_streaming_amd import edge0 as E
    S, seed = G.QWEN3_MOE, 0
    ds = _qwen3_stack(S, seed)
    ds.stack.set_mode(E.EDGE0_STACK_PERSISTENT)
    report, rels = _run(ds, S, seed, 4, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[stack] qwen3moe persistent: worst rel-L2 {max(rels):.3e}, median "
          f"{np.median(rels):.3e}, waived {report.count('waived')}/{len(report)}")
    ds.stack.close()


def test_persistent_mode_rejects_unsupported_shape(torch_cuda):
    """The tiny layer shape (d_model 256) is outside the persistent path:
    EDGE0_EINVAL and the graph mode stays in force."""
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S = G.TINY
    ds = DeviceStack(S, G.StackGen(S, 1), 4, (1, 2), (2, 3), log=None)
    with pytest.raises(E.Edge0Error) as ei:
        ds.stack.set_mode(E.EDGE0_STACK_PERSISTENT)
    assert ei.value.code == E.EDGE0_EINVAL
    with pytest.raises(E.Edge0Error):
        ds.stack.set_mode(7)


def test_persistent_mode_bounded_wait_reports_error(torch_cuda):
    """A workgroup that waits past the spin limit at a grid boundary records
    EDGE0_EHIP, raises the abort word and leaves; every other workgroup exits
    on seeing it.  Forced from the host with a limit of one poll, on a
    4-layer stack of Qwen3-MoE-shaped layers; the launch must end (no hang)
    and report the error."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE
    ds = DeviceStack(S, G.StackGen(S, 5), 4, (1, 2), (2, 3), log=None)
    ds.stack.set_mode(E.EDGE0_STACK_PERSISTENT)
    ds.stack.set_spin_limit(1)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    ds.step(to_device(G.stack_hidden(S, 5, 0)), h_out, 0)
    torch.cuda.synchronize()
    assert ds.stack.error() == E.EDGE0_EHIP
    with pytest.raises(E.Edge0Error):
        ds.stack.set_spin_limit(-1)
    ds.stack.close()
