"""Throughput of the streaming-MoE decode hot path on one MI355X.

The headline (D2): one step = one decode token through 40 Qwen3-MoE-shaped
layers (hidden 2048, 128 experts, inter 768, K = 4, int4 group 64, per-expert
LoRA r=16 a=32, prerouter heads at layers 6..37, prediction-routed layers
7..38), all expert bundles resident in HBM, a fresh seeded hidden state per
step.  The same JSON line carries the other measurement rows under "rows":

  d0     the tiny layer (hidden 256, 16 experts): one layer call = router +
         MoE layer + prerouter head, 10^4 back-to-back calls, us per call
  d1_k4, d1_k8
         one Qwen3-MoE-shaped layer at K = 4 and 8: the MoE layer call and
         the head call, over 64 layer instances (128 heads) in distinct HBM
         addresses, rotated so the 256 MB memory-side cache holds no earlier
         call's weights; replayed as HIP graphs; median of 5 runs x 1024 calls
  d3     the stack over a 3 GiB slot pool staged from pinned host memory:
         prediction arm, on-demand arm (fill kernel and DMA copies), the
         closed loop (routing from the device) and all-resident, 5 rounds in
         rotated order, medians
  d4     the grouped multi-token layer (K = 8) at 1, 4, 8, 16, 32 tokens per
         call on the rotated instances
  prefill the whole-layer prefill call at 512, 2048 and 4096 tokens (K = 8)
  merge  merge-and-requantise of one layer's experts: retention of the LoRA
         delta in the weights and in the layer's outputs
  files  the d3 stack with the pool filled from per-layer expert files on
         disk (O_DIRECT, and the page cache), the raw read rate as roofline

Every row has a roofline object and the oracle timed on this host's cores
(1 thread and all threads) on a bounded sample.

  python bench.py [--gpus 1] [--steps 256] [--warmup 16] [--no-cpu] [--rows all|none]
  python bench.py --workload streamed|files|grouped|layer|tiny|prefill|merge   (one row alone)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s (batch 1, 40-layer MoE stack) + achieved HBM GB/s vs peak"
# HBM traffic of one k_layer_fused launch from two rocprofv3 --pmc passes over
# this workload (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), scaled by what
# the same counters read for a device copy of known size (256 MiB copy:
# FETCH_SIZE 131084.7 KiB -> x2.0, WRITE_SIZE 262144 KiB -> x1.0).  Valid only
# for the kernel sources it was taken on (hash below); otherwise None.
TRAFFIC_RECORD = {"src_sha": "af617369d9b2ef8e", "fetch_kib": 3884.8, "write_kib": 54.1,
                  "fetch_scale": 2.0, "write_scale": 1.0}
KERNEL_SOURCES = ("common.h", "moe_internal.h", "gemv_dev.h", "heads_dev.h", "moe.hip")
# the same two counters for k_merge_mfma<16, 4> (one Qwen3-MoE-shaped expert),
# valid for the merge source they were taken on
MERGE_TRAFFIC_RECORD = {"src_sha": "e4afe3fcf46594bb", "fetch_kib": 1677.8, "write_kib": 2646.0,
                        "fetch_scale": 2.0, "write_scale": 1.0}
HBM_PEAK_GBPS = 8000.0
N_LAYERS, OWNERS, CONSUMERS = 40, (6, 37), (7, 38)


# ------------------------------------------------------------------ bytes
def bundle_alg_bytes(S):
    """One expert's int4 gate/up/down rows with their bf16 scales and biases."""
    d, I, g = S.d_model, S.d_inter, S.group
    return 3 * I * d // 2 + 3 * (I * d // g) * 2 * 2


def lora_alg_bytes(S):
    """One expert's six bf16 LoRA factors."""
    d, I, r = S.d_model, S.d_inter, S.lora_rank
    return 2 * (r * d + I * r) * 2 + (r * I + d * r) * 2


def head_alg_bytes(S):
    """One head call: fc1 hidden-state columns, the 2K gathered one-hot rows,
    fc2, the linear residual and the biases (fp16)."""
    d, E, K, H = S.d_model, S.n_experts, S.top_k, S.head_hidden
    return H * d * 2 + 2 * K * H * 2 + E * H * 2 + E * d * 2 + H * 2 + E * 2


def moe_alg_bytes(S):
    """One MoE layer call: the K routed experts' bundles and adapters."""
    return S.top_k * (bundle_alg_bytes(S) + lora_alg_bytes(S))


def step_bytes(S, n_routers):
    """Algorithmic HBM bytes of one decode step (every weight byte the step
    must read once): K bundles + adapters per layer, 32 heads and the plain
    routers that run."""
    n_heads = OWNERS[1] - OWNERS[0] + 1
    return N_LAYERS * moe_alg_bytes(S) + n_heads * head_alg_bytes(S) + \
        n_routers * S.n_experts * S.d_model * 2


def fused_bytes(S):
    """Algorithmic bytes of one k_layer_fused launch (prediction-routed
    layer: input + gate/up): the K experts' gate and up int4 rows with scales
    and biases, their LoRA A_gate/A_up rows, the previous layer's h and
    fixed-point y, and what it writes (h, y, x, the cleared accumulator, the
    gate/up rows before their LoRA terms as fp32, and t = A x).  The LoRA B
    terms, the SwiGLU and A_down h are the down launch's."""
    d, I, K, g, r = S.d_model, S.d_inter, S.top_k, S.group, S.lora_rank
    w = K * 2 * (I * d // 2 + 2 * I * (d // g) * 2)
    lora = K * 2 * r * d * 2
    reads = d * 2 + d * 8
    writes = 3 * d * 2 + d * 8 + K * 2 * I * 4 + K * 2 * r * 4
    return w + lora + reads + writes


def flow_bytes(S, n_routers):
    """Algorithmic bytes of the persistent layers launch of one step (every
    layer's K bundles and adapters, the plain routers that run, and each
    layer's input/output activations: x, y, h written, the fixed-point y
    read and cleared); the heads run after it as their own launches."""
    d = S.d_model
    act = 3 * d * 2 + 2 * d * 8
    return N_LAYERS * (moe_alg_bytes(S) + act) + n_routers * S.n_experts * d * 2


def xlayer_bytes(S):
    """Algorithmic bytes of one k_xlayer launch of a prediction-routed layer:
    the K routed experts' bundles and adapters, read once; the previous
    layer's h and fixed-point y read; x, y, h and the fixed-point y written."""
    d = S.d_model
    return moe_alg_bytes(S) + d * 2 + d * 8 + 3 * d * 2 + d * 8


def merge_traffic():
    """Counter-derived HBM bytes per k_merge_mfma launch, or None if merge.hip
    changed since the counters were taken."""
    import hashlib
    with open(os.path.join(ROOT, "int4_expert_streaming_amd", "csrc", "merge.hip"), "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()[:16]
    r = MERGE_TRAFFIC_RECORD
    if h != r["src_sha"]:
        return None
    return int((r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"]) * 1024)


def gate_up_traffic():
    """Counter-derived HBM bytes per k_layer_fused launch, or None if the
    kernel sources changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "int4_expert_streaming_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    r = TRAFFIC_RECORD
    if not r["src_sha"] or h.hexdigest()[:16] != r["src_sha"]:
        return None
    return int((r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"]) * 1024)


def roofline(kernel, nbytes, us):
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
            "bytes_per_launch": int(nbytes), "avg_launch_us": round(us, 3)}


# ----------------------------------------------------------- CPU baseline
def host_info():
    """The host the oracle is timed on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"os_cpu_count": os.cpu_count(), "nproc": nproc, "model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _pool_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])


def oracle_timed(unit, budget_s):
    """unit() runs one unit of oracle work and returns the seconds its timed
    part took.  Repeated within budget_s, once with the BLAS pool limited to
    one thread and once at its own size; returns (s per unit at 1 thread,
    s per unit at all threads, threads, units per pass)."""
    from threadpoolctl import threadpool_limits
    out = []
    for limit in (1, None):
        with threadpool_limits(limits=limit):
            ts, t0 = [], time.time()
            while not ts or (time.time() - t0 < budget_s and len(ts) < 64):
                ts.append(unit())
        out.append((float(np.mean(ts)), len(ts)))
    return out[0][0], out[1][0], _pool_threads(), min(out[0][1], out[1][1])


def cpu_record(value_1, value_n, unit, threads, sample):
    return {"value": round(value_n, 6), "unit": unit, "cores": int(threads), "kind": "oracle",
            "single_thread_value": round(value_1, 6), "host": host_info(), "sample": sample}


def cpu_baseline_stack(S, seed, budget_s=8.0):
    """D2: the oracle's plain router + top-K, MoE layer over K experts and
    prerouter head on layers of the same stack, extrapolated to one 40-layer
    step (32 heads, 8 routers)."""
    import oracle as O
    from synth import gen as G
    scale = S.lora_alpha / S.lora_rank
    layers = list(range(OWNERS[0], OWNERS[1] + 1))
    state = {"i": 0}

    def unit():
        L = layers[state["i"] % len(layers)]
        state["i"] += 1
        x = G.stack_hidden(S, seed, 10_000 + L)
        wr, head = G.router_weight(S, seed, L), G.head_tensors(S, seed, L)
        t0 = time.perf_counter()
        ids, w = O.softmax_topk(O.router_logits(wr, x), S.top_k)
        t_r = time.perf_counter() - t0
        ex = {int(e): G.expert_tensors(S, seed, L, int(e)) for e in ids}
        lo = {int(e): G.lora_tensors(S, seed, L, int(e)) for e in ids}
        t0 = time.perf_counter()
        O.moe_layer(ex, ids, w, x, S.group, lo, scale)
        t_m = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.prerouter_commit(head, x, ids, None, S.n_experts, S.top_k)
        t_h = time.perf_counter() - t0
        return N_LAYERS * t_m + 32 * t_h + 8 * t_r
    s1, sn, thr, n = oracle_timed(unit, budget_s)
    return cpu_record(1.0 / s1, 1.0 / sn, "tok/s", thr,
                      f"{n} stack layers per thread setting (router + top-K, MoE K={S.top_k}, "
                      f"head) timed, each extrapolated to a 40-layer step; "
                      f"{sn:.2f} s/step at all threads, {s1:.2f} s/step at 1")


# ------------------------------------------------------------- D0: tiny
def row_tiny(args, log):
    """The tiny layer: router + MoE layer + head per call, 10^4 calls."""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import SlotPoolBuffer, head_to_device, to_device
    S = G.TINY
    sh = E.make_shape(S)
    En, K = S.n_experts, S.top_k
    pool = SlotPoolBuffer(sh, En)
    for e in range(En):
        pool.load(e, G.expert_tensors(S, args.seed, 0, e), G.lora_tensors(S, args.seed, 0, e))
    table = torch.arange(En, dtype=torch.int32, device="cuda")
    wr = to_device(G.router_weight(S, args.seed, 0))
    head_d = head_to_device(G.head_tensors(S, args.seed, 0))  # kept alive: the head points at it
    head = E.make_head(head_d)
    ws = E.new_workspace(sh)
    x = to_device(G.hidden(S, args.seed, 0))
    y = torch.empty_like(x)
    ids = torch.zeros(K, dtype=torch.int32, device="cuda")
    w = torch.zeros(K, dtype=torch.float32, device="cuda")
    pids = [torch.arange(K, dtype=torch.int32, device="cuda") for _ in range(2)]
    pw = torch.zeros(K, dtype=torch.float32, device="cuda")

    def call(i):
        E.edge0_router(sh, wr, x, None, ids, w, ws)
        E.edge0_moe_layer(sh, pool.pool, table, ids, w, x, y, ws)
        E.edge0_prerouter(sh, head, x, ids, pids[(i + 1) & 1], None, pids[i & 1], pw, ws)

    for i in range(200):
        call(i)
    torch.cuda.synchronize()
    # issued call by call from the host (the binding's overhead included)
    n = 10_000
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    ev0.record(stream)
    for i in range(n):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - h0) * 1e6 / n
    issued_us = ev0.elapsed_time(ev1) * 1e3 / n
    # the device's own latency: 1000 calls captured as one graph, 10 replays
    y_ref = y.clone()
    us, runs = _graph_time(torch, call, 1000, runs=10)
    assert torch.equal(y, y_ref), "graph replay differs from the host-issued calls"
    assert E.edge0_workspace_error(ws) == 0
    nbytes = moe_alg_bytes(S) + head_alg_bytes(S) + En * S.d_model * 2
    log(f"[d0] tiny layer call {us:.2f} us in a graph; issued from the host {issued_us:.2f} us "
        f"(host {host_us:.2f} us)")
    out = {"metric": "tiny layer call latency (router + MoE + head)", "value": round(us, 3),
           "unit": "us/call", "higher_is_better": False,
           "config": {"workload": "tiny MoE layer: hidden 256, 16 experts, inter 128, K=4, "
                                  "group 32, LoRA r=8, head 288->64->16 + residual",
                      "timing": "HIP graph of 1000 back-to-back calls, median of 10 replays; "
                                f"also {n} calls issued one by one from the host"},
           "graph_runs_us": runs, "host_issued_us_per_call": round(issued_us, 3),
           "host_issue_us_per_call": round(host_us, 3),
           "roofline": roofline("router + MoE layer + head (one call)", nbytes, us)}
    out["roofline"]["note"] = "latency-bound by design (0.37 MB per call)"
    if not args.no_cpu:
        import oracle as O
        wr_h, head_h = G.router_weight(S, args.seed, 0), G.head_tensors(S, args.seed, 0)
        ex = {e: G.expert_tensors(S, args.seed, 0, e) for e in range(En)}
        lo = {e: G.lora_tensors(S, args.seed, 0, e) for e in range(En)}
        xh = G.hidden(S, args.seed, 0)

        def unit():
            t0 = time.perf_counter()
            i_, w_ = O.softmax_topk(O.router_logits(wr_h, xh), K)
            O.moe_layer(ex, i_, w_, xh, S.group, lo, S.lora_alpha / S.lora_rank)
            O.prerouter_commit(head_h, xh, i_, None, En, K)
            return time.perf_counter() - t0
        s1, sn, thr, reps = oracle_timed(unit, 2.0)
        out["cpu_baseline"] = cpu_record(s1 * 1e6, sn * 1e6, "us/call", thr,
                                         f"{reps} single calls per thread setting")
    return out


# -------------------------------------------- rotated Qwen3-MoE instances
class Instances:
    """n_inst copies of n_gen generated Qwen3-MoE-shaped layers (all E
    experts each) at distinct HBM addresses, plus n_heads head copies, so
    that rotating over them defeats the 256 MB memory-side cache."""

    def __init__(self, S, seed, log, n_gen=8, n_inst=64, n_heads=128):
        import torch
        from synth import gen as G
        from int4_expert_streaming_amd import edge0 as E
        from int4_expert_streaming_amd.stackbuild import pack_layer
        from int4_expert_streaming_amd.weights import SlotPoolBuffer, head_to_device, to_device
        self.S, self.n_gen, self.n_inst = S, n_gen, n_inst
        En = S.n_experts
        sh = E.make_shape(S)
        gen = G.StackGen(S, seed)
        self.pool = SlotPoolBuffer(sh, n_inst * En)
        bb = self.pool.slot_bytes
        t0 = time.time()
        for L in range(n_gen):
            parts = [(gen.expert(L, e), gen.lora(L, e)) for e in range(En)]
            pack_layer(sh, parts, lambda e: self.pool.slot_ptr(L * En + e))
        for i in range(n_gen, n_inst):
            src = (i % n_gen) * En * bb
            self.pool.mem[i * En * bb:(i + 1) * En * bb].copy_(self.pool.mem[src:src + En * bb])
        self.tables = [torch.arange(i * En, (i + 1) * En, dtype=torch.int32, device="cuda")
                       for i in range(n_inst)]
        self.routers = [to_device(gen.router(L)) for L in range(n_gen)]
        base = [head_to_device(gen.head(L)) for L in range(n_gen)]
        self.heads_d = [{k: (None if v is None else v.clone()) for k, v in base[i % n_gen].items()}
                        for i in range(n_heads)]
        self.heads = [E.make_head(h) for h in self.heads_d]
        torch.cuda.synchronize()
        log(f"[instances] {n_inst} layers x {En} experts + {n_heads} heads "
            f"({self.pool.mem.numel() / 1e9:.1f} GB) in {time.time() - t0:.1f}s")


def _graph_time(torch, body, n_calls, runs=5, check=None):
    """Median us per call of `body(c)` for c in 0..n_calls-1, captured as one
    HIP graph and replayed `runs` times (after one untimed replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(8):
            body(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in range(n_calls):
            body(c)
    g.replay()
    torch.cuda.synchronize()
    if check is not None:
        check()
    times = []
    for _ in range(runs):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) * 1e3 / n_calls)
    if check is not None:
        check()
    return float(np.median(times)), [round(t, 3) for t in times]


def row_layer(args, log, inst, K):
    """D1: one Qwen3-MoE-shaped layer at K: the MoE layer call, the head call
    and the two together, rotated over the instances."""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = inst.S.with_k(K)
    sh = E.make_shape(S)
    En, d, n_inst = S.n_experts, S.d_model, inst.n_inst
    n_heads = len(inst.heads)
    ws = E.new_workspace(sh)
    xs = [to_device(G.hidden(S, 700 + i)) for i in range(n_heads)]
    ids, ws_w = [], []
    for i in range(n_inst):  # routing of each instance: its router's top-K
        a = torch.zeros(K, dtype=torch.int32, device="cuda")
        b = torch.zeros(K, dtype=torch.float32, device="cuda")
        E.edge0_router(sh, inst.routers[i % inst.n_gen], xs[i], None, a, b, ws)
        ids.append(a)
        ws_w.append(b)
    rng = np.random.default_rng(args.seed + K)
    prev = [torch.from_numpy(rng.choice(En, K, replace=False).astype(np.int32)).cuda()
            for _ in range(n_heads)]
    ys = [torch.empty(d, dtype=torch.int16, device="cuda") for _ in range(n_inst)]
    pid = torch.zeros(K, dtype=torch.int32, device="cuda")
    pw = torch.zeros(K, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def moe(c):
        i = c % n_inst
        E.edge0_moe_layer(sh, inst.pool.pool, inst.tables[i], ids[i], ws_w[i], xs[i], ys[i], ws)

    def head(c):
        i = c % n_heads
        E.edge0_prerouter(sh, inst.heads[i], xs[i], ids[i % n_inst], prev[i], None, pid, pw, ws)

    def both(c):
        head(c)
        moe(c)

    # graph replays against an eager call of the same instance: bit-identical y
    ref = torch.empty(d, dtype=torch.int16, device="cuda")
    E.edge0_moe_layer(sh, inst.pool.pool, inst.tables[5], ids[5], ws_w[5], xs[5], ref, ws)
    torch.cuda.synchronize()

    def check():
        assert torch.equal(ys[5], ref), "graph replay differs from the eager call"

    n_calls = 1024
    us_moe, runs_moe = _graph_time(torch, moe, n_calls, check=check)
    us_head, runs_head = _graph_time(torch, head, n_calls)
    us_both, _ = _graph_time(torch, both, n_calls)
    assert E.edge0_workspace_error(ws) == 0
    b_moe, b_head = moe_alg_bytes(S), head_alg_bytes(S)
    log(f"[d1] K={K}: MoE {us_moe:.2f} us ({b_moe / us_moe / 1e3:.0f} GB/s), head {us_head:.2f} us "
        f"({b_head / us_head / 1e3:.0f} GB/s), both {us_both:.2f} us")
    out = {"metric": f"one Qwen3-MoE-shaped layer, K={K}: MoE layer call GB/s vs peak",
           "value": round(b_moe / (us_moe * 1e-6) / 1e9, 1), "unit": "GB/s",
           "higher_is_better": True,
           "config": {"workload": f"one Qwen3-MoE-shaped layer, 1 token, K={K}, "
                                  f"{n_inst} rotated layer instances, {n_heads} heads",
                      "d_model": d, "n_experts": En, "d_inter": S.d_inter, "top_k": K,
                      "group": S.group, "lora_rank": S.lora_rank, "head_hidden": S.head_hidden,
                      "timing": f"HIP graph of {n_calls} calls, median of 5 replays"},
           "moe_us_per_call": round(us_moe, 3), "moe_runs_us": runs_moe,
           "head_us_per_call": round(us_head, 3), "head_runs_us": runs_head,
           "head_plus_moe_us_per_call": round(us_both, 3),
           "moe_bytes": b_moe, "head_bytes": b_head,
           "head_gbps": round(b_head / (us_head * 1e-6) / 1e9, 1),
           "head_plus_moe_gbps": round((b_moe + b_head) / (us_both * 1e-6) / 1e9, 1),
           "roofline": roofline("edge0_moe_layer (fused layer input + LoRA A x + int4 gate/up, int4 down with the LoRA epilogue, combine)",
                                b_moe, us_moe)}
    if not args.no_cpu:
        import oracle as O
        gen = G.StackGen(S, args.seed)
        x = G.hidden(S, 700)
        idh = ids[0].cpu().numpy()
        wh = ws_w[0].cpu().numpy().astype(np.float64)
        ex = {int(e): gen.expert(0, int(e)) for e in idh}
        lo = {int(e): gen.lora(0, int(e)) for e in idh}
        hd = gen.head(0)

        def unit():
            t0 = time.perf_counter()
            O.moe_layer(ex, idh, wh, x, S.group, lo, S.lora_alpha / S.lora_rank)
            O.prerouter_commit(hd, x, idh, None, En, K)
            return time.perf_counter() - t0
        s1, sn, thr, reps = oracle_timed(unit, 3.0)
        out["cpu_baseline"] = cpu_record(
            (b_moe + b_head) / s1 / 1e9, (b_moe + b_head) / sn / 1e9, "GB/s", thr,
            f"{reps} single layer calls (MoE K={K} + head) per thread setting: "
            f"{sn * 1e3:.1f} ms at all threads, {s1 * 1e3:.1f} ms at 1")
    return out


# ----------------------------------------------------------- D4: grouped
def row_grouped(args, log, inst):
    """Grouped multi-token layer (K = 8) at 1, 4, 8, 16 and 32 tokens per
    call, Zipf(1.1) routing, rotated over the instances."""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = inst.S.with_k(8)
    sh = E.make_shape(S)
    En, K, d, I, r = S.n_experts, S.top_k, S.d_model, S.d_inter, S.lora_rank
    n_inst = inst.n_inst
    bb = bundle_alg_bytes(S) + lora_alg_bytes(S)
    gws = E.new_grouped_workspace(sh)
    stream = torch.cuda.current_stream()
    results = {}
    for T in (1, 4, 8, 16, 32):
        routes = [G.grouped_routing(En, K, T, seed=args.seed * 1000 + 17 * T + i,
                                    layer=i % inst.n_gen) for i in range(n_inst)]
        ids = [to_device(rt[0]) for rt in routes]
        wts = [torch.from_numpy(rt[1]).cuda() for rt in routes]
        xs = [to_device(G.hidden(S, 500 + T * 100 + i, n=T)) for i in range(n_inst)]
        y = torch.empty((T, d), dtype=torch.int16, device="cuda")
        union = float(np.mean([np.count_nonzero(np.bincount(rt[0].ravel(), minlength=En))
                               for rt in routes]))

        def timed(flags, n_calls=256):
            for i in range(32):
                E.edge0_moe_grouped(sh, inst.pool.pool, inst.tables[i % n_inst], T,
                                    ids[i % n_inst], wts[i % n_inst], xs[i % n_inst], y, gws, flags)
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for c in range(n_calls):
                i = c % n_inst
                E.edge0_moe_grouped(sh, inst.pool.pool, inst.tables[i], T, ids[i], wts[i], xs[i],
                                    y, gws, flags)
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) * 1e3 / n_calls

        us = float(np.median([timed(0) for _ in range(5)]))
        if args.mfma_sweep:
            sweep = {"gemv_only": round(timed(E.EDGE0_GROUPED_NO_MFMA), 2)}
            for mn in (2, 4, 8, 24):
                sweep[f"mfma_from_{mn}"] = round(timed(E.grouped_mfma_min(mn)), 2)
            log(f"[d4] T={T} us/call by MFMA threshold: default {us:.2f}, {sweep}")
        nbytes = union * bb
        flops = 2.0 * T * K * (3 * d * I + 2 * r * d + 2 * I * r + r * I + d * r)
        results[T] = {"us_per_call": round(us, 2), "tok_s": round(T / (us * 1e-6), 1),
                      "experts": round(union, 2),
                      "path": "mfma tiles" if T >= 3 else "gemv",
                      "union_bytes": int(nbytes), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                      "tflops": round(flops / (us * 1e-6) / 1e12, 3)}
        log(f"[d4] T={T}: {results[T]}")
    best = results[32]
    out = {"metric": "grouped MoE layer tok/s (K=8, Qwen3-MoE shapes) + union-bytes GB/s vs peak",
           "value": best["tok_s"], "unit": "tok/s", "higher_is_better": True,
           "config": {"workload": "one Qwen3-MoE-shaped layer, 1-32 tokens per call, K=8, "
                                  f"Zipf(1.1) routing, {n_inst} rotated layer instances",
                      "timing": "median of 5 runs of 256 calls"},
           "roofline": roofline("edge0_moe_grouped at T=32 (bucketing + int4 MFMA tiles)",
                                best["union_bytes"], best["us_per_call"]),
           "per_tokens": {str(k): v for k, v in results.items()}}
    if not args.no_cpu:
        import oracle as O
        gen = G.StackGen(S, args.seed)
        T = 4
        idg, wg = G.grouped_routing(En, K, T, seed=args.seed * 1000 + 17 * T, layer=0)
        xg = G.hidden(S, 500 + T * 100, n=T)
        ex = {int(e): gen.expert(0, int(e)) for e in np.unique(idg)}
        lo = {int(e): gen.lora(0, int(e)) for e in np.unique(idg)}

        def unit():
            t0 = time.perf_counter()
            O.grouped_layer(ex, idg, wg.astype(np.float64), xg, S.group, lo,
                            S.lora_alpha / S.lora_rank)
            return time.perf_counter() - t0
        s1, sn, thr, reps = oracle_timed(unit, 3.0)
        out["cpu_baseline"] = cpu_record(T / s1, T / sn, "tok/s", thr,
                                         f"{reps} grouped calls of {T} tokens (K=8) per thread "
                                         "setting, per token as the oracle defines it")
    return out


# ----------------------------------------------------------- f3: prefill
def row_prefill(args, log, inst):
    """Whole-layer prefill: one Qwen3-MoE-shaped layer (K = 8, Zipf(1.1)
    routing) at 512, 2048 and 4096 tokens per call, rotated over the
    instances; every expert of the layer is hit."""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = inst.S.with_k(8)
    sh = E.make_shape(S)
    En, K, d, I, r = S.n_experts, S.top_k, S.d_model, S.d_inter, S.lora_rank
    n_inst = inst.n_inst
    bb = bundle_alg_bytes(S) + lora_alg_bytes(S)
    Tmax = 4096
    pws = E.new_prefill_workspace(sh, Tmax)
    stream = torch.cuda.current_stream()
    results = {}
    for T in (512, 2048, 4096):
        n_rot = 8  # routing/input sets, instance c % n_inst
        routes = [G.grouped_routing(En, K, T, seed=args.seed * 1000 + 31 * T + i, layer=i)
                  for i in range(n_rot)]
        ids = [to_device(rt[0]) for rt in routes]
        wts = [torch.from_numpy(rt[1]).cuda() for rt in routes]
        xs = [to_device(G.hidden(S, 900 + T + i, n=T)) for i in range(n_rot)]
        y = torch.empty((T, d), dtype=torch.int16, device="cuda")
        union = float(np.mean([np.count_nonzero(np.bincount(rt[0].ravel(), minlength=En))
                               for rt in routes]))

        def run(n_calls):
            for c in range(n_calls):
                i, q = c % n_inst, c % n_rot
                E.edge0_moe_prefill(sh, inst.pool.pool, inst.tables[i], T, ids[q], wts[q], xs[q],
                                    y, pws, Tmax)
        run(4)
        torch.cuda.synchronize()
        times = []
        n_calls = 16 if T <= 512 else 8
        for _ in range(5):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            run(n_calls)
            ev1.record(stream)
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) * 1e3 / n_calls)
        us = float(np.median(times))
        nbytes = union * bb
        flops = 2.0 * T * K * (3 * d * I + 2 * r * d + 2 * I * r + r * I + d * r)
        results[T] = {"us_per_call": round(us, 1), "tok_s": round(T / (us * 1e-6), 1),
                      "experts": round(union, 2), "expert_bytes": int(nbytes),
                      "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                      "frac_of_bf16_mfma_peak": round(flops / (us * 1e-6) / 2.5e15, 4)}
        log(f"[prefill] T={T}: {results[T]}")
    assert E.edge0_workspace_error(pws) == 0
    best = results[4096]
    out = {"metric": "whole-layer prefill tok/s (one Qwen3-MoE-shaped layer, K=8)",
           "value": best["tok_s"], "unit": "tok/s", "higher_is_better": True,
           "config": {"workload": "one Qwen3-MoE-shaped layer, 512 / 2048 / 4096 tokens per call, "
                                  f"K=8, Zipf(1.1) routing, {n_inst} rotated layer instances",
                      "timing": "median of 5 runs"},
           "roofline": {"kernel": "edge0_moe_prefill at 4096 tokens (LDS-staged int4 GEMMs on bf16 MFMA over 64-pair tiles)",
                        "bound": "mfma", "achieved": best["tflops"], "peak": 2500.0,
                        "unit": "TFLOP/s", "frac": round(best["tflops"] / 2500.0, 4),
                        "traffic": None, "avg_launch_us": best["us_per_call"]},
           "per_tokens": {str(k): v for k, v in results.items()}}
    if not args.no_cpu:
        import oracle as O
        gen = G.StackGen(S, args.seed)
        T = 4
        idp, wp = G.grouped_routing(En, K, T, seed=5, layer=0)
        xp = G.hidden(S, 906, n=T)
        ex = {int(e): gen.expert(0, int(e)) for e in np.unique(idp)}
        lo = {int(e): gen.lora(0, int(e)) for e in np.unique(idp)}

        def unit():
            t0 = time.perf_counter()
            O.grouped_layer(ex, idp, wp.astype(np.float64), xp, S.group, lo,
                            S.lora_alpha / S.lora_rank)
            return time.perf_counter() - t0
        s1, sn, thr, reps = oracle_timed(unit, 3.0)
        out["cpu_baseline"] = cpu_record(T / s1, T / sn, "tok/s", thr,
                                         f"{reps} calls of {T} tokens (K=8) per thread setting; "
                                         "the oracle defines prefill token by token")
    return out


# ------------------------------------------------------- f4: merge/requant
def row_merge(args, log, inst):
    """Merge-and-requantise every expert of one Qwen3-MoE-shaped layer: the
    weight-level retention per projection over the layer, the output-level
    retention 1 - |U - M| / |U - B| of layer calls on 64 tokens (U with the
    unmerged LoRA, M on the merged experts, B on the base alone), and the
    merge kernel's time."""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import to_device
    S = inst.S
    sh = E.make_shape(S)
    sh0 = E.make_shape(S)
    sh0.lora_rank = 0
    En, d, I, g, r = S.n_experts, S.d_model, S.d_inter, S.group, S.lora_rank
    bb0 = int(E.edge0_bundle_layout_of(sh0).bytes)
    merged = torch.zeros(En * bb0, dtype=torch.uint8, device="cuda")
    stats = torch.zeros((En, 6), dtype=torch.float64, device="cuda")
    mws = torch.empty(E.lib.edge0_merge_workspace_bytes(E.C.byref(sh)), dtype=torch.uint8,
                      device="cuda")
    def merge_one(c):  # layer instance 0, expert c
        e = c % En
        E.edge0_merge_requant(sh, inst.pool.slot_ptr(e), merged[e * bb0:(e + 1) * bb0], stats[e], mws)

    # one call per expert, captured as a graph (issued one by one from Python
    # the calls would measure the host, not the kernels)
    us, us_runs = _graph_time(torch, merge_one, En)
    st = stats.cpu().numpy().sum(axis=0)
    ret = {p: round(float(st[2 * i] / st[2 * i + 1]), 4) for i, p in enumerate(("gate", "up", "down"))}
    # output level: 64 tokens through the layer three ways
    ws = E.new_workspace(sh)
    pool0 = E.SlotPool(merged.data_ptr(), bb0, En)
    table = torch.arange(En, dtype=torch.int32, device="cuda")
    U, M, B = [], [], []
    rng = np.random.default_rng(args.seed + 41)
    for i in range(64):
        x = to_device(G.hidden(S, 5000 + i))
        ids = torch.from_numpy(rng.choice(En, S.top_k, replace=False).astype(np.int32)).cuda()
        wv = rng.uniform(0.1, 1.0, S.top_k)
        w = torch.from_numpy((wv / wv.sum()).astype(np.float32)).cuda()
        outs = []
        for shp, pool in ((sh, inst.pool.pool), (sh0, pool0), (sh0, inst.pool.pool)):
            y = torch.zeros(d, dtype=torch.int16, device="cuda")
            E.edge0_moe_layer(shp, pool, table, ids, w, x, y, ws)
            outs.append(y)
        torch.cuda.synchronize()
        for lst, y in zip((U, M, B), outs):
            lst.append(y.cpu().numpy().view(np.uint16))
    f = lambda a: (np.asarray(a, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    Uf, Mf, Bf = f(np.stack(U)), f(np.stack(M)), f(np.stack(B))
    out_ret = 1.0 - float(np.linalg.norm(Uf - Mf) / np.linalg.norm(Uf - Bf))
    # ALU work: per element of the three projections, the r-term delta (2r)
    # and the requantisation (8); HBM bytes: the codes read and written, the
    # group scales and biases read and written, the LoRA factors read
    n_el = 3 * d * I
    flops = n_el * (2 * r + 8)
    hbm_bytes = 2 * (n_el // 2) + 2 * 2 * 2 * (n_el // g) + 2 * 3 * r * (d + I)
    log(f"[merge] {us:.1f} us per expert; weight retention {ret}; output retention {out_ret:.4f}")
    out = {"metric": "merge-and-requantise: weight-level retention of the LoRA delta per projection",
           "value": ret, "unit": "fraction of sum(delta^2)", "higher_is_better": True,
           "config": {"workload": "every expert of one Qwen3-MoE-shaped layer (128), LoRA r=16 "
                                  "alpha=32 merged into int4 group 64 and requantised",
                      "output_retention_tokens": 64,
                      "timing": "HIP graph of 128 calls (one per expert), median of 5 replays"},
           "output_retention": round(out_ret, 4),
           "us_per_expert": round(us, 2), "us_runs": us_runs,
           "roofline": {"kernel": "k_merge_mfma + k_merge_sum (one expert)", "bound": "alu",
                        "achieved": round(flops / (us * 1e-6) / 1e12, 3), "peak": 157.3,
                        "unit": "TFLOP/s", "frac": round(flops / (us * 1e-6) / 1e12 / 157.3, 4),
                        "traffic": merge_traffic(), "traffic_kernel": "k_merge_mfma only",
                        "avg_launch_us": round(us, 2),
                        "hbm_bytes_per_expert": hbm_bytes,
                        "hbm_gbps": round(hbm_bytes / (us * 1e-6) / 1e9, 1),
                        "note": "fp32 count: 2r + 8 per weight element (the delta's 2r run on "
                                "the matrix cores); at the vector peak this floor, 1.2 us, is "
                                "above the HBM floor, 0.7 us"}}
    if not args.no_cpu:
        import oracle as O
        gen = G.StackGen(S, args.seed)
        ex, lo = gen.expert(0, 0), gen.lora(0, 0)

        def unit():
            t0 = time.perf_counter()
            for p in ("gate", "up", "down"):
                O.merge_requant(ex[p + "_q"], ex[p + "_s"], ex[p + "_b"], lo["a_" + p],
                                lo["b_" + p], S.lora_alpha / r, g)
            return time.perf_counter() - t0
        s1, sn, thr, reps = oracle_timed(unit, 3.0)
        out["cpu_baseline"] = cpu_record(1e6 * s1, 1e6 * sn, "us/expert", thr,
                                         f"{reps} experts merged by the oracle per thread setting")
    return out


# ------------------------------------------------------------ D3: staged
def h2d_bandwidth(host_mem, nbytes, n=128):
    """Pinned host -> device copy rate (GB/s) for n copies of nbytes each on
    one stream: the host-link roofline of the staged arms."""
    import torch
    dst = torch.empty(nbytes * 8, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(8):  # warm
            dst[(i % 8) * nbytes:(i % 8 + 1) * nbytes].copy_(host_mem[i * nbytes:(i + 1) * nbytes],
                                                              non_blocking=True)
        ev0.record(stream)
        for i in range(n):
            j = i % 8
            dst[j * nbytes:(j + 1) * nbytes].copy_(host_mem[i * nbytes:(i + 1) * nbytes],
                                                   non_blocking=True)
        ev1.record(stream)
    torch.cuda.synchronize()
    return n * nbytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9


def stage_kernel_bandwidth(S, host, n_layers, n_sets=24):
    """Rate (GB/s) of the stager's fill kernel alone: n_sets requests of K
    fresh bundles each on one stream, nothing else running."""
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.weights import SlotPoolBuffer
    sh = E.make_shape(S)
    K = S.top_k
    pool = SlotPoolBuffer(sh, n_sets * K)
    table = torch.full((n_layers, S.n_experts), -1, dtype=torch.int32, device="cuda")
    sg = E.Stager(sh, pool.pool, n_layers, host.ptrs, table)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(n_sets):
        L = i % n_layers
        ids = [(K * (i // n_layers) + k) % S.n_experts for k in range(K)]
        sg.stage(L, i // n_layers, ids, stream)
        sg.release(L, i // n_layers, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    nbytes = sg.stats()["bytes_staged"]
    sg.close()
    return nbytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9


STAGED_ARMS = ("ahead", "demand", "ahead_dma", "demand_dma", "loop", "resident")


def row_staged(args, log, rounds=5, warmup=16, steps=64):
    """The 40-layer stack over a 3 GiB HBM slot pool filled from pinned host
    bundles.  Arms (each a fresh pool: cold start), in rotated order over
    `rounds` rounds on the same host tier:
      ahead / ahead_dma   prediction arm over a Zipf(1.1) trace (~25 %
                          adjacent-token overlap): the next step's predicted
                          sets staged on a side stream (fill kernel / DMA)
      demand / demand_dma each set filled right after its router
      loop                the closed loop: routing from the device (router
                          top-K, the heads' predictions read back once per
                          step and staged); random heads, so its routing
                          statistics are the heads' own
      resident            every bundle in HBM, the same launches: the
                          compute-only step time"""
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import (HostBundles, StreamedStack,
                                                       device_routers_heads)
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE
    gen = G.StackGen(S, args.seed)
    host = HostBundles(S, gen, N_LAYERS, log=log)
    routers, heads = device_routers_heads(gen, N_LAYERS, range(OWNERS[0], OWNERS[1] + 1))
    bb = host.bundle_bytes
    n_slots = (3 << 30) // bb
    total = warmup + steps
    trace = G.zipf_trace(S.n_experts, S.top_k, N_LAYERS, total + 1, args.seed, keep_p=0.06)
    overlap = float(np.mean([len(set(trace[t, L]) & set(trace[t - 1, L])) / S.top_k
                             for t in range(1, total) for L in range(N_LAYERS)]))
    trace_dev = torch.from_numpy(trace).cuda()
    h0 = to_device(np.stack([G.stack_hidden(S, args.seed, t) for t in range(total)]))
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    bw_dma = h2d_bandwidth(host.mem, bb)
    bw_kernel = stage_kernel_bandwidth(S, host, N_LAYERS)
    bw = max(bw_dma, bw_kernel)
    log(f"[d3] host link: DMA copies {bw_dma:.1f} GB/s, fill kernel {bw_kernel:.1f} GB/s "
        f"({bb}-byte bundles); trace overlap {overlap:.3f}")
    per_arm = {a: [] for a in STAGED_ARMS}
    for rnd in range(rounds):
        k = rnd % len(STAGED_ARMS)
        order = STAGED_ARMS[k:] + STAGED_ARMS[:k]
        for arm in order:
            slots = N_LAYERS * S.n_experts if arm == "resident" else n_slots
            ss = StreamedStack(S, gen, N_LAYERS, OWNERS, CONSUMERS, slots, log=None, host=host,
                               routers=routers, heads=heads)
            if arm.endswith("_dma"):
                ss.stager.set_copy_mode(1)
            if arm == "resident":  # every bundle staged before timing
                for L in range(N_LAYERS):
                    for e0 in range(0, S.n_experts, 16):
                        ss.stager.stage(L, 1 << 20, list(range(e0, e0 + 16)))
                        ss.stager.release(L, 1 << 20)
                ss.stager.flush()
                torch.cuda.synchronize()
            mode = {"loop": E.EDGE0_STAGE_LOOP}.get(arm, not arm.startswith("demand"))

            def step(t):
                if arm == "loop":
                    E.stack_step_staged(ss.stack, ss.stager, h0[t], h_out, t, None, None, None,
                                        mode, ss.copy_stream)
                else:
                    ss.step(h0[t], h_out, t, trace_dev[t], trace[t], trace[t + 1], mode)
            stream = torch.cuda.current_stream()
            for t in range(warmup):
                step(t)
            torch.cuda.synchronize()
            st0 = ss.stager.stats()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for t in range(warmup, total):
                step(t)
            ev1.record(stream)
            torch.cuda.synchronize()
            st1 = ss.stager.stats()
            ms = ev0.elapsed_time(ev1) / steps
            dd = {k_: st1[k_] - st0[k_] for k_ in st1}
            rec = {"ms_per_step": ms, "hit_rate": dd["hits"] / max(1, dd["touches"]),
                   "misses_per_step": dd["misses"] / steps,
                   "h2d_bytes_per_step": dd["bytes_staged"] / steps}
            if arm == "loop":
                ids = ss.stack.buffers()["ids"].cpu().numpy()
                rec["distinct_experts_last_step"] = int(len(np.unique(ids)))
            per_arm[arm].append(rec)
            del ss
            torch.cuda.synchronize()
        log(f"[d3] round {rnd}: " + ", ".join(f"{a} {per_arm[a][-1]['ms_per_step']:.3f} ms"
                                              for a in STAGED_ARMS))
    arms = {}
    for a, recs in per_arm.items():
        med = {k_: float(np.median([r[k_] for r in recs])) for k_ in recs[0]}
        arms[a] = {"ms_per_step": round(med["ms_per_step"], 4),
                   "tok_s": round(1000.0 / med["ms_per_step"], 2),
                   "rounds_ms": [round(r["ms_per_step"], 4) for r in recs],
                   "hit_rate": round(med["hit_rate"], 4),
                   "misses_per_step": round(med["misses_per_step"], 2),
                   "h2d_bytes_per_step": int(med["h2d_bytes_per_step"])}
        if "distinct_experts_last_step" in med:
            arms[a]["distinct_experts_last_step"] = int(med["distinct_experts_last_step"])
    t_comp = arms["resident"]["ms_per_step"]
    for a in STAGED_ARMS[:-1]:
        r = arms[a]
        copy_ms = r["h2d_bytes_per_step"] / (bw * 1e9) * 1e3
        exposed = max(0.0, r["ms_per_step"] - t_comp)
        r["copy_ms_per_step"] = round(copy_ms, 4)
        r["exposed_wait_ms_per_step"] = round(exposed, 4)
        r["overlap"] = round(1.0 - exposed / copy_ms, 4) if copy_ms > 0 else None
        r["host_link_ceiling_tok_s"] = round(1000.0 / copy_ms, 2) if copy_ms > 0 else None
    a = arms["ahead"]
    achieved = a["h2d_bytes_per_step"] / (a["ms_per_step"] * 1e-3) / 1e9
    out = {"metric": "staged decode tok/s (batch 1, 40-layer MoE stack, 3 GiB HBM pool)",
           "value": a["tok_s"], "unit": "tok/s", "higher_is_better": True,
           "config": {"workload": "40-layer Qwen3-MoE-shaped decode stack, experts staged from "
                                  "pinned host memory into a 3 GiB HBM pool (LRU)",
                      "n_slots": n_slots, "bundle_bytes": bb, "top_k": S.top_k,
                      "trace": "Zipf(1.1), per-layer permutation, keep_p 0.06",
                      "trace_overlap": round(overlap, 4),
                      "timing": f"{rounds} rounds, arm order rotated, {warmup} warmup + "
                                f"{steps} timed steps per arm and round, medians"},
           "h2d_gbps": {"dma_copy": round(bw_dma, 2), "fill_kernel": round(bw_kernel, 2)},
           "roofline": {"kernel": "host link (prediction arm's H2D bytes per step)",
                        "bound": "host-link", "achieved": round(achieved, 2),
                        "peak": round(bw, 2), "unit": "GB/s", "frac": round(achieved / bw, 4),
                        "traffic": None},
           "arms": arms}
    out_files = None
    if args.rows_files:
        try:
            out_files = row_files(args, log, S, gen, host, routers, heads, trace, trace_dev, h0,
                                  h_out)
        except Exception as e:  # the disk tier must not cost the other rows their line
            log(f"[files] not measured: {e!r}")
            out_files = {"skipped": repr(e)}
    if not args.no_cpu:
        import oracle as O
        own, con = range(OWNERS[0], OWNERS[1] + 1), range(CONSUMERS[0], CONSUMERS[1] + 1)
        ev = O.canonical_requests(total, N_LAYERS, own, con, heads_at_end=True)
        t0 = time.perf_counter()
        O.lru_replay(ev, lambda L, t: trace[t, L], n_slots)
        s = (time.perf_counter() - t0) / total
        out["cpu_baseline"] = cpu_record(1e3 * s, 1e3 * s, "ms/step (LRU replay)", 1,
                                         f"the oracle LRU replay of {total} steps of the trace "
                                         "(single-threaded Python)")
    del host
    return out, out_files


def direct_read_gbps(paths, record_bytes, n_threads=16, seconds=3.0):
    """Raw O_DIRECT read rate of the layer files (GB/s): n_threads threads
    reading whole records chosen uniformly at random over every file (the
    widest access pattern; the arms re-read Zipf-hot records), the disk
    tier's roofline."""
    import mmap
    import threading
    fds = [os.open(p, os.O_RDONLY | os.O_DIRECT) for p in paths]
    n_rec = (os.fstat(fds[0]).st_size - 4096) // record_bytes
    done = [0] * n_threads
    stop = time.time() + seconds

    def work(i):
        buf = mmap.mmap(-1, record_bytes)
        rng = np.random.default_rng(i)
        while time.time() < stop:
            fd = fds[int(rng.integers(len(fds)))]
            os.preadv(fd, [buf], 4096 + int(rng.integers(n_rec)) * record_bytes)
            done[i] += record_bytes
    t0 = time.time()
    th = [threading.Thread(target=work, args=(i,)) for i in range(n_threads)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    for fd in fds:
        os.close(fd)
    return sum(done) / (time.time() - t0) / 1e9


FILE_ARMS = ("ahead_file", "demand_file", "loop_file", "ahead_pagecache")


def row_files(args, log, S, gen, host, routers, heads, trace, trace_dev, h0, h_out, rounds=2,
              warmup=8, steps=24):
    """The staged stack with the 3 GiB pool filled from per-layer expert files
    on the box's disk (the SSD tier under the pinned host pool): the
    prediction arm, the on-demand arm and the closed loop reading with
    O_DIRECT, and the prediction arm through the page cache (warm), rotated
    over `rounds` rounds; the raw O_DIRECT read rate is the roofline."""
    import shutil
    import tempfile
    import torch
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import StreamedStack, write_layer_files
    base_dir = os.environ.get("EDGE0_FILE_DIR", "/tmp")
    need = len(host.ptrs) * int(E.lib.edge0_layer_file_record_bytes(E.C.byref(E.make_shape(S))))
    free = shutil.disk_usage(base_dir).free
    if free < need + (4 << 30):
        return {"skipped": f"{free / 1e9:.1f} GB free under {base_dir}, the files need "
                           f"{need / 1e9:.1f} GB"}
    d = tempfile.mkdtemp(prefix="e0_layers_", dir=base_dir)
    try:
        paths = write_layer_files(host, d, S.n_experts, log=log)
        sh = E.make_shape(S)
        rec = int(E.lib.edge0_layer_file_record_bytes(E.C.byref(sh)))
        ssd = direct_read_gbps(paths, rec)
        n_slots = (3 << 30) // host.bundle_bytes
        log(f"[files] O_DIRECT read rate {ssd:.2f} GB/s ({rec}-byte records, random, 16 threads)")
        per_arm = {a: [] for a in FILE_ARMS}
        total = warmup + steps
        for rnd in range(rounds):
            k = rnd % len(FILE_ARMS)
            for arm in FILE_ARMS[k:] + FILE_ARMS[:k]:
                ft = E.FileTier(sh, paths, n_buffers=64, n_threads=8,
                                direct=not arm.endswith("pagecache"))
                ss = StreamedStack(S, gen, N_LAYERS, OWNERS, CONSUMERS, n_slots, log=None,
                                   host=host, routers=routers, heads=heads, files=ft)
                mode = E.EDGE0_STAGE_LOOP if arm.startswith("loop") else arm.startswith("ahead")

                def step(t):
                    if arm.startswith("loop"):
                        E.stack_step_staged(ss.stack, ss.stager, h0[t], h_out, t, None, None, None,
                                            mode, ss.copy_stream)
                    else:
                        ss.step(h0[t], h_out, t, trace_dev[t], trace[t], trace[t + 1], mode)
                for t in range(warmup):
                    step(t)
                torch.cuda.synchronize()
                st0, f0 = ss.stager.stats(), ft.stats()
                t0 = time.perf_counter()
                for t in range(warmup, total):
                    step(t)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) * 1e3 / steps
                st1, f1 = ss.stager.stats(), ft.stats()
                dd = {k_: st1[k_] - st0[k_] for k_ in st1}
                fb, fns = f1["bytes"] - f0["bytes"], f1["read_ns"] - f0["read_ns"]
                per_arm[arm].append({"ms_per_step": ms,
                                     "hit_rate": dd["hits"] / max(1, dd["touches"]),
                                     "misses_per_step": dd["misses"] / steps,
                                     "file_bytes_per_step": fb / steps,
                                     "read_gbps": fb / max(1, fns)})
                del ss
                ft.close()
                torch.cuda.synchronize()
            log(f"[files] round {rnd}: " + ", ".join(f"{a} {per_arm[a][-1]['ms_per_step']:.1f} ms"
                                                      for a in FILE_ARMS))
        arms = {}
        for a, recs in per_arm.items():
            med = {k_: float(np.median([r[k_] for r in recs])) for k_ in recs[0]}
            arms[a] = {"ms_per_step": round(med["ms_per_step"], 3),
                       "tok_s": round(1000.0 / med["ms_per_step"], 2),
                       "rounds_ms": [round(r["ms_per_step"], 3) for r in recs],
                       "hit_rate": round(med["hit_rate"], 4),
                       "misses_per_step": round(med["misses_per_step"], 2),
                       "file_bytes_per_step": int(med["file_bytes_per_step"]),
                       "read_gbps_in_batches": round(med["read_gbps"], 2),
                       "ssd_ceiling_tok_s": round(ssd * 1e9 / max(1.0, med["file_bytes_per_step"]), 2)}
        a = arms["ahead_file"]
        achieved = a["file_bytes_per_step"] / (a["ms_per_step"] * 1e-3) / 1e9
        return {"metric": "staged decode tok/s from expert files (batch 1, 40-layer MoE stack, "
                          "3 GiB HBM pool, O_DIRECT)",
                "value": a["tok_s"], "unit": "tok/s", "higher_is_better": True,
                "config": {"workload": "40-layer Qwen3-MoE-shaped decode stack, experts read from "
                                       "per-layer files on the box's disk into a 3 GiB HBM pool",
                           "trace": "as the staged row (Zipf(1.1), overlap 0.25)",
                           "timing": f"{rounds} rounds, arm order rotated, {warmup} warmup + "
                                     f"{steps} timed steps per arm and round, host wall clock, "
                                     "medians",
                           "file_dir_fs": "ext4 virtio disk of the box (df of the directory)"},
                "direct_read_gbps": round(ssd, 2),
                "roofline": {"kernel": "disk reads (prediction arm's file bytes per step)",
                             "bound": "ssd", "achieved": round(achieved, 2), "peak": round(ssd, 2),
                             "unit": "GB/s", "frac": round(achieved / ssd, 4), "traffic": None},
                "arms": arms}
    finally:
        shutil.rmtree(d, ignore_errors=True)


# ------------------------------------------------------------ D2: stack
def row_stack(args, log):
    import torch
    from synth import gen as G
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE
    ds = DeviceStack(S, G.StackGen(S, args.seed), N_LAYERS, OWNERS, CONSUMERS, log=log)
    mode_name = args.stack_mode
    if mode_name != "graphs":
        try:
            ds.stack.set_mode({"persistent": E.EDGE0_STACK_PERSISTENT, "xcd": E.EDGE0_STACK_XCD,
                               "xlayer": E.EDGE0_STACK_XLAYER}[mode_name])
        except E.Edge0Error as e:
            log(f"[bench] {mode_name} mode unavailable ({e}); using per-layer graphs")
            mode_name = "graphs"
    persistent = mode_name in ("persistent", "xcd")
    sched = {"folded": E.EDGE0_HEADS_FOLDED, "after": E.EDGE0_HEADS_AFTER_LAYERS}
    ds.stack.set_head_schedule(sched[args.head_schedule])
    total = args.warmup + args.steps
    h0 = to_device(np.stack([G.stack_hidden(S, args.seed, t) for t in range(total)]))
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    for t in range(args.warmup):
        ds.step(h0[t], h_out, t)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for t in range(args.warmup, total):
        ds.step(h0[t], h_out, t)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = 1000.0 / ms_step
    sbytes = step_bytes(S, n_routers=8)
    step_gbps = sbytes * tok_s / 1e9
    ds.stack.set_timing(1)
    if persistent:
        # dominant kernel: the one launch that runs all 40 layers, bracketed
        # by events on the launching stream over further steps
        k_ms = []
        for t in range(total, total + 8):
            ds.step(h0[t % total], h_out, t)
            k_ms += ds.stack.kernel_ms()
        k_name = ("k_xstep" if mode_name == "xcd" else "k_flow_step") + \
            " (all 40 layers: routing, int4 gate/up + LoRA + SwiGLU, down, combine)"
        k_bytes = flow_bytes(S, n_routers=8)
        k_traffic = None
    else:
        # dominant kernel: the prediction-routed layers' first launch (32 per
        # step), timed by events the dispatch records at its start and end on
        # the launching stream, over further steps of the same stack
        k_ms = []
        for t in range(total, total + 8):
            ds.step(h0[t % total], h_out, t)
            per_layer = ds.stack.kernel_ms()
            k_ms += [per_layer[L] for L in range(CONSUMERS[0], CONSUMERS[1] + 1)]
        if mode_name == "xlayer":
            k_name = ("k_xlayer (one whole layer: input, int4 gate/up + LoRA + SwiGLU, XCD-local "
                      "hand-off of h, int4 down + LoRA, combine)")
            k_bytes = xlayer_bytes(S)
            k_traffic = None
        else:
            k_name = "k_layer_fused (layer input + LoRA A x + int4 gate/up GEMV; the LoRA B terms and SwiGLU follow in the down launch)"
            k_bytes = fused_bytes(S)
            k_traffic = gate_up_traffic()
    ds.stack.set_timing(0)
    other_sched = None
    if mode_name == "graphs" and not args.no_head_ab:
        # the other head schedule on the same stack, same step count
        other = "after" if args.head_schedule == "folded" else "folded"
        ds.stack.set_head_schedule(sched[other])
        t0 = total + 8
        for t in range(t0, t0 + args.warmup):
            ds.step(h0[t % total], h_out, t)
        torch.cuda.synchronize()
        ev0.record(stream)
        for t in range(t0 + args.warmup, t0 + args.warmup + args.steps):
            ds.step(h0[t % total], h_out, t)
        ev1.record(stream)
        torch.cuda.synchronize()
        other_sched = {"schedule": other, "ms_per_step": round(ev0.elapsed_time(ev1) / args.steps, 5)}
        ds.stack.set_head_schedule(sched[args.head_schedule])
        log(f"[bench] heads {other}: {other_sched['ms_per_step'] * 1000:.1f} us/step")
    k_mean = float(np.mean(k_ms))
    k_gbps = k_bytes / (k_mean * 1e-3) / 1e9
    log(f"[bench] {ms_step * 1000:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), "
        f"{step_gbps:.0f} GB/s step, {k_name.split()[0]} {k_mean * 1000:.2f} us = {k_gbps:.0f} GB/s")
    rl = roofline(k_name, k_bytes, k_mean * 1000)
    rl["traffic"] = k_traffic
    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "40-layer Qwen3-MoE-shaped decode stack, all experts resident",
                   "stack_mode": mode_name,
                   "head_schedule": args.head_schedule if mode_name == "graphs" else "after",
                   "d_model": S.d_model, "n_experts": S.n_experts, "d_inter": S.d_inter,
                   "top_k": S.top_k, "group": S.group, "lora_rank": S.lora_rank,
                   "head_hidden": S.head_hidden, "layers": N_LAYERS, "heads": "6-37",
                   "prediction_routed": "7-38", "global_batch": 1, "parallelism": "none"},
        "step_bytes": sbytes, "step_gbps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "roofline": rl,
    }
    if other_sched is not None:
        out["other_head_schedule"] = other_sched
    del ds
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def single_row_line(row, args):
    """A row run alone: its own JSON line in the contract's keys."""
    out = {"metric": row["metric"], "value": row["value"], "unit": row["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
           "higher_is_better": row.get("higher_is_better", True), "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    out.update({k: v for k, v in row.items() if k not in out})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--rows", choices=["all", "none"], default="all",
                    help="all: the headline line also carries rows d0, d1_k4, d1_k8, d3, d4")
    ap.add_argument("--workload", choices=["resident", "streamed", "grouped", "layer", "tiny",
                                           "prefill", "merge", "files"],
                    default="resident",
                    help="resident: the headline (40-layer stack, every bundle in HBM); the "
                         "others run one row alone: streamed (d3), grouped (d4), layer (d1), "
                         "tiny (d0)")
    ap.add_argument("--stack-mode", choices=["graphs", "persistent", "xcd", "xlayer"],
                    default="graphs",
                    help="resident workload: per-layer launches replayed as HIP graphs (the "
                         "default, the fastest here), the layers as one persistent launch per "
                         "step, the XCD-split persistent launch, or one XCD-split launch per "
                         "layer")
    ap.add_argument("--head-schedule", choices=["folded", "after"], default="after",
                    help="graphs mode: the heads batched after the last layer (default) or "
                         "their fc1 rows beside the down launches; the other is timed too for "
                         "comparison")
    ap.add_argument("--no-head-ab", action="store_true",
                    help="do not time the other head schedule (profiling runs)")
    ap.add_argument("--mfma-sweep", action="store_true",
                    help="grouped row: also time other MFMA thresholds")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (hardware counter "
                         "calibration: known bytes moved) and exit")
    ap.add_argument("--no-files", action="store_true",
                    help="skip the expert-file row (writes 15 GB of layer files to EDGE0_FILE_DIR, "
                         "default /tmp)")
    args = ap.parse_args()
    args.rows_files = (not args.no_files) or args.workload == "files"
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 4}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    import torch
    torch.cuda.set_device(0)
    from synth import gen as G
    if args.workload in ("streamed", "files"):
        d3, files_row = row_staged(args, log)
        print(json.dumps(single_row_line(d3 if args.workload == "streamed" else files_row, args)),
              flush=True)
        return
    if args.workload in ("grouped", "layer", "prefill", "merge"):
        inst = Instances(G.QWEN3_MOE, args.seed, log)
        if args.workload in ("grouped", "prefill", "merge"):
            row = {"grouped": row_grouped, "prefill": row_prefill,
                   "merge": row_merge}[args.workload](args, log, inst)
            print(json.dumps(single_row_line(row, args)), flush=True)
        else:
            for K in (4, 8):
                print(json.dumps(single_row_line(row_layer(args, log, inst, K), args)), flush=True)
        return
    if args.workload == "tiny":
        print(json.dumps(single_row_line(row_tiny(args, log), args)), flush=True)
        return

    out = row_stack(args, log)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline_stack(G.QWEN3_MOE, args.seed)
    if args.rows == "all":
        t0 = time.time()
        rows = {}

        def row(name, fn, *a):
            # a row that fails is recorded as such; the headline line still prints
            try:
                rows[name] = fn(*a)
            except Exception as e:
                log(f"[bench] row {name} not measured: {e!r}")
                rows[name] = {"failed": repr(e)}
        row("d0", row_tiny, args, log)
        try:
            inst = Instances(G.QWEN3_MOE, args.seed, log)
        except Exception as e:
            log(f"[bench] layer instances not built: {e!r}")
            inst = None
        if inst is not None:
            row("d1_k4", row_layer, args, log, inst, 4)
            row("d1_k8", row_layer, args, log, inst, 8)
            row("d4", row_grouped, args, log, inst)
            row("prefill", row_prefill, args, log, inst)
            row("merge", row_merge, args, log, inst)
            del inst
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        row("d3", row_staged, args, log)
        if isinstance(rows.get("d3"), tuple):
            rows["d3"], files_row = rows["d3"]
            if files_row is not None:
                rows["files"] = files_row
        out["rows"] = rows
        log(f"[bench] rows measured in {time.time() - t0:.0f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
