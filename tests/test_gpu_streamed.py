"""GPU parity of the staged decode stack (edge0_stager_* and
edge0_stack_step_staged) against the oracle.

Routing comes from a seeded Zipf trace; each layer's weights are the softmax
of its own logits taken at the trace ids (plain router, or - prediction arm,
step > 0, prediction-routed layer - the logits its owner's head produced at
the previous step).  After every step:
  * the device slot table equals the oracle LRU replay's resident map for
    the same canonical request order, bit-exact, and the stager's counters
    equal the replay's;
  * every resident slot holds the bytes of its host bundle;
  * every checked layer matches the oracle teacher-forced (the GPU's hidden
    state entering the layer): x, weights (rel 1e-5), y (rel-L2 2e-3), h."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import REL_L2_MAX, W_REL_MAX, check_bf16_rounding, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _resident(events, ids_of, n_slots, n_layers, n_experts):
    """The oracle's id -> slot map after the events, as a [L][E] table."""
    recs, tot = O.lru_replay(events, ids_of, n_slots)
    owner = {}
    for r in recs:
        for e, s in zip(r["ids"], r["slots"]):
            owner[s] = (r["L"], e)
    table = np.full((n_layers, n_experts), -1, np.int32)
    for s, (L, e) in owner.items():
        table[L, e] = s
    return table, tot


def _streamed_stack(S, gen, n_layers, owners, consumers, n_slots, source, tmp_dir):
    """The staged stack with its misses from pinned host bundles (source
    "host") or from layer files written from them, read with O_DIRECT
    ("file_direct") or through the page cache ("file_cached")."""
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import HostBundles, StreamedStack, write_layer_files
    if source == "host":
        return StreamedStack(S, gen, n_layers, owners, consumers, n_slots, log=None)
    host = HostBundles(S, gen, n_layers, log=None)
    paths = write_layer_files(host, str(tmp_dir), S.n_experts)
    ft = E.FileTier(E.make_shape(S), paths, n_buffers=32, n_threads=4,
                    direct=source == "file_direct")
    return StreamedStack(S, gen, n_layers, owners, consumers, n_slots, log=None, host=host,
                         files=ft)


def _run(S, seed, n_layers, owners, consumers, n_slots, steps, ahead, layers_of, keep_p=0.1,
         copy_mode=0, free_bias=False, source="host", tmp_dir=None):
    import torch
    from int4_expert_streaming_amd.weights import to_device
    gen = G.StackGen(S, seed, free_bias=free_bias)
    En, K = S.n_experts, S.top_k
    ss = _streamed_stack(S, gen, n_layers, owners, consumers, n_slots, source, tmp_dir)
    ss.stager.set_copy_mode(copy_mode)
    trace = G.zipf_trace(En, K, n_layers, steps + 1, seed + 100, keep_p=keep_p)
    trace_dev = torch.from_numpy(trace).cuda()
    own = range(owners[0], owners[1] + 1) if ahead else range(0)
    con = range(consumers[0], consumers[1] + 1) if ahead else range(0)
    ids_of = lambda L, t: trace[t, L]
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    router = {L: gen.router(L) for L in range(n_layers)}
    head = {L: gen.head(L) for L in own}
    prev_x = None
    worst = 0.0
    for t in range(steps):
        print(f"[streamed] ahead={ahead} step {t}", flush=True)
        h0 = G.stack_hidden(S, seed, t)
        ss.step(to_device(h0), h_out, t, trace_dev[t], trace[t], trace[t + 1] if ahead else None,
                ahead)
        torch.cuda.synchronize()
        # slot table and counters against the replay of the same requests
        ev = O.canonical_requests(t + 1, n_layers, own, con, heads_at_end=True)
        want, tot = _resident(ev, ids_of, n_slots, n_layers, En)
        got = ss.table.cpu().numpy()
        assert np.array_equal(got, want), (t, np.argwhere(got != want)[:8])
        st = ss.stager.stats()
        assert (st["hits"], st["misses"]) == (tot["hits"], tot["misses"]), (st, tot)
        assert st["bytes_staged"] == st["misses"] * ss.host.bundle_bytes
        # resident slots hold their bundles
        pool = ss.pool.mem.view(n_slots, -1)
        for L, e in zip(*np.nonzero(want >= 0)):
            if (L + e + t) % 7 == 0 or S.d_model <= 256:
                s = int(want[L, e])
                assert torch.equal(pool[s].cpu(), ss.host.bundle(int(L), int(e), En)), (L, e, s)
        # layers, teacher-forced
        b = ss.stack.buffers()
        snap = {k: v.cpu().numpy() for k, v in b.items()}
        hh, xx, yy = (snap[k].view(np.uint16) for k in ("h", "x", "y"))
        assert np.array_equal(hh[0], h0)
        assert np.array_equal(snap["ids"], trace[t])
        for L in layers_of(t):
            check_bf16_rounding(xx[L], O.rmsnorm(O.bf16_to_f64(hh[L])))
            ids = trace[t, L]
            if ahead and L in con and t > 0:
                logits = O.prerouter_logits(head[L - 1], prev_x[L - 1], trace[t - 1, L - 1],
                                            trace[t - 2, L - 1] if t >= 2 else None, En)
            else:
                logits = O.router_logits(router[L], xx[L])
            w_o = O.softmax_at(logits, ids)
            assert np.max(np.abs(snap["w"][L] - w_o) / np.abs(w_o)) <= W_REL_MAX, (L, t)
            ex = {int(e): gen.expert(L, int(e)) for e in ids}
            lo = {int(e): gen.lora(L, int(e)) for e in ids}
            y_o = O.moe_layer(ex, ids, w_o, xx[L], S.group, lo, S.lora_alpha / S.lora_rank)
            rel = rel_l2(O.bf16_to_f64(yy[L]), y_o)
            worst = max(worst, rel)
            assert rel <= REL_L2_MAX, (L, t, rel)
            h_next = O.f64_to_bf16_bits(O.bf16_to_f64(hh[L]) + O.bf16_to_f64(yy[L]))
            assert np.array_equal(h_next, hh[L + 1]), (L, t)
        prev_x = xx.copy()
    return ss, worst


@pytest.mark.parametrize("ahead,copy_mode", [(True, 0), (False, 0), (True, 1), (False, 1)])
def test_small_streamed_stack_every_layer(torch_cuda, ahead, copy_mode):
    """10 tiny layers, a 40-slot pool (160 bundles: constant eviction); both
    arms, fills by the copy kernel (0) or by DMA copies (1)."""
    ss, worst = _run(G.TINY, 5, 10, (2, 7), (3, 8), 40, 6, ahead, lambda t: range(10),
                     copy_mode=copy_mode)
    print(f"[streamed] tiny ahead={ahead} mode={copy_mode}: worst rel-L2 {worst:.3e}, "
          f"{ss.stager.stats()}")


@pytest.mark.timeout(900)
def test_qwen3moe_streamed_stack_every_layer(torch_cuda):
    """12 Qwen3-MoE-shaped layers over a 64-slot pool (at most 36 pinned),
    prediction arm: evictions from the second step on; every layer of 4
    steps, with group biases drawn independently of the scales."""
    ss, worst = _run(G.QWEN3_MOE, 1, 12, (2, 9), (3, 10), 64, 4, True, lambda t: range(12),
                     keep_p=0.06, free_bias=True)
    assert ss.stager.stats()["evictions"] > 0
    print(f"[streamed] qwen3moe: worst rel-L2 {worst:.3e}, {ss.stager.stats()}")


@pytest.mark.parametrize("ahead", [True, False])
def test_small_streamed_stack_free_bias(torch_cuda, ahead):
    """The tiny staged stack with group biases independent of the scales."""
    ss, worst = _run(G.TINY, 6, 10, (2, 7), (3, 8), 40, 4, ahead, lambda t: range(10),
                     free_bias=True)
    print(f"[streamed] tiny free bias ahead={ahead}: worst rel-L2 {worst:.3e}")


def test_stager_rejects_pageable_host_memory(torch_cuda):
    """Host bundles must be pinned (device-readable); pageable memory is
    refused at create, before any copy could touch it."""
    import numpy as np
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import SlotPoolBuffer
    sh = E.make_shape(G.TINY)
    bb = int(E.edge0_bundle_layout_of(sh).bytes)
    pageable = np.zeros(2 * G.TINY.n_experts * bb, np.uint8)
    ptrs = [pageable.ctypes.data + k * bb for k in range(2 * G.TINY.n_experts)]
    pool = SlotPoolBuffer(sh, 4)
    table = torch.full((2, G.TINY.n_experts), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(E.Edge0Error) as ei:
        E.Stager(sh, pool.pool, 2, ptrs, table)
    assert ei.value.code == E.EDGE0_EINVAL
    # a pinned buffer is accepted
    pinned = torch.zeros(2 * G.TINY.n_experts * bb, dtype=torch.uint8, pin_memory=True)
    sg = E.Stager(sh, pool.pool, 2, [pinned.data_ptr() + k * bb for k in range(2 * G.TINY.n_experts)],
                  table)
    sg.close()


def _run_loop(S, seed, n_layers, owners, consumers, n_slots, steps, source="host", tmp_dir=None):
    """The closed loop (EDGE0_STAGE_LOOP): no trace; router layers commit
    their own top-K, prediction-routed layers execute what their owner's
    head committed one step earlier, and those predictions are what the
    host staged.  Checked after every step: the executed routing of a
    prediction-routed layer is the previous step's prediction; each
    commit against the oracle's on the oracle's logits (near-tie waivers);
    the slot table and counters against the LRU replay of the executed and
    predicted sets; every layer teacher-forced."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    from tests.layer_setup import check_routing
    gen = G.StackGen(S, seed)
    En, K = S.n_experts, S.top_k
    ss = _streamed_stack(S, gen, n_layers, owners, consumers, n_slots, source, tmp_dir)
    own = range(owners[0], owners[1] + 1)
    con = range(consumers[0], consumers[1] + 1)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    router = {L: gen.router(L) for L in range(n_layers)}
    head = {L: gen.head(L) for L in own}
    executed, predicted = {}, {}   # step -> [L][K]
    prev_x = None
    stats = []
    for t in range(steps):
        print(f"[streamed] loop step {t}", flush=True)
        h0 = G.stack_hidden(S, seed, t)
        E.stack_step_staged(ss.stack, ss.stager, to_device(h0), h_out, t, None, None, None,
                            E.EDGE0_STAGE_LOOP, ss.copy_stream)
        torch.cuda.synchronize()
        b = ss.stack.buffers()
        snap = {k: v.cpu().numpy() for k, v in b.items()}
        executed[t], predicted[t] = snap["ids"].copy(), snap["pred_ids"].copy()
        hh, xx, yy = (snap[k].view(np.uint16) for k in ("h", "x", "y"))
        assert np.array_equal(hh[0], h0)
        for L in range(n_layers):
            ids = executed[t][L]
            assert len(set(ids.tolist())) == K and ids.min() >= 0 and ids.max() < En
            if L in con and t > 0:
                # prediction-as-routing: the staged (predicted) set is the routed set
                assert np.array_equal(ids, predicted[t - 1][L]), (L, t)
                logits = O.prerouter_logits(head[L - 1], prev_x[L - 1], executed[t - 1][L - 1],
                                            executed[t - 2][L - 1] if t >= 2 else None, En)
            else:
                logits = O.router_logits(router[L], xx[L])
            stats.append(check_routing(ids, snap["w"][L], logits, K))
            check_bf16_rounding(xx[L], O.rmsnorm(O.bf16_to_f64(hh[L])))
            w_o = O.softmax_at(logits, ids)
            assert np.max(np.abs(snap["w"][L] - w_o) / np.abs(w_o)) <= W_REL_MAX, (L, t)
            ex = {int(e): gen.expert(L, int(e)) for e in ids}
            lo = {int(e): gen.lora(L, int(e)) for e in ids}
            y_o = O.moe_layer(ex, ids, w_o, xx[L], S.group, lo, S.lora_alpha / S.lora_rank)
            assert rel_l2(O.bf16_to_f64(yy[L]), y_o) <= REL_L2_MAX, (L, t)
            h_next = O.f64_to_bf16_bits(O.bf16_to_f64(hh[L]) + O.bf16_to_f64(yy[L]))
            assert np.array_equal(h_next, hh[L + 1]), (L, t)
        # the predictions of this step, against the oracle's commit
        for L in own:
            lo_ = O.prerouter_logits(head[L], xx[L], executed[t][L],
                                     executed[t - 1][L] if t >= 1 else None, En)
            stats.append(check_routing(predicted[t][L + 1], snap["pred_w"][L + 1], lo_, K))
        # slot table and counters: the replay of the executed sets and, after
        # the step, the predicted sets of the next one
        ids_of = lambda L, s: executed[s][L] if s in executed else predicted[s - 1][L]
        ev = O.canonical_requests(t + 1, n_layers, own, con, heads_at_end=True)
        want, tot = _resident(ev, ids_of, n_slots, n_layers, En)
        got = ss.table.cpu().numpy()
        assert np.array_equal(got, want), (t, np.argwhere(got != want)[:8])
        st = ss.stager.stats()
        assert (st["hits"], st["misses"]) == (tot["hits"], tot["misses"]), (st, tot)
        prev_x = xx.copy()
    assert stats.count("exact") >= 0.9 * len(stats), stats.count("waived")
    return ss


def test_small_streamed_stack_closed_loop(torch_cuda):
    """10 tiny layers over a 40-slot pool, 6 steps, routing from the device."""
    ss = _run_loop(G.TINY, 7, 10, (2, 7), (3, 8), 40, 6)
    print(f"[streamed] tiny loop: {ss.stager.stats()}")


@pytest.mark.timeout(900)
def test_qwen3moe_streamed_stack_closed_loop(torch_cuda):
    """12 Qwen3-MoE-shaped layers over a 64-slot pool, 4 steps, routing
    from the device (router layers' own top-K, the heads' predictions)."""
    ss = _run_loop(G.QWEN3_MOE, 2, 12, (2, 9), (3, 10), 64, 4)
    print(f"[streamed] qwen3moe loop: {ss.stager.stats()}")


@pytest.mark.parametrize("source,ahead,copy_mode", [("file_direct", True, 0),
                                                    ("file_direct", False, 1),
                                                    ("file_cached", True, 1)])
def test_small_streamed_stack_from_files(torch_cuda, tmp_path, source, ahead, copy_mode):
    """The tiny staged stack with every miss read from the layer files (with
    O_DIRECT or through the page cache) into pinned staging buffers, then
    copied by the fill kernel or DMA: the same checks as from host memory."""
    ss, worst = _run(G.TINY, 5, 10, (2, 7), (3, 8), 40, 6, ahead, lambda t: range(10),
                     copy_mode=copy_mode, source=source, tmp_dir=tmp_path)
    st = ss.files.stats()
    assert st["reads"] == ss.stager.stats()["misses"] and st["bytes"] > 0
    print(f"[streamed] tiny from files ({source}) ahead={ahead}: worst rel-L2 {worst:.3e}, {st}")


@pytest.mark.timeout(900)
def test_qwen3moe_streamed_from_files_and_loop(torch_cuda, tmp_path):
    """12 Qwen3-MoE-shaped layers over a 64-slot pool from O_DIRECT layer
    files: the trace arm for 4 steps, then the closed loop for 3."""
    ss, worst = _run(G.QWEN3_MOE, 1, 12, (2, 9), (3, 10), 64, 4, True, lambda t: range(12),
                     keep_p=0.06, source="file_direct", tmp_dir=tmp_path / "a")
    assert ss.stager.stats()["evictions"] > 0
    ss = _run_loop(G.QWEN3_MOE, 2, 12, (2, 9), (3, 10), 64, 3, source="file_direct",
                   tmp_dir=tmp_path / "b")
    print(f"[streamed] qwen3moe from files: worst rel-L2 {worst:.3e}, {ss.files.stats()}")
