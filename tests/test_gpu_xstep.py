"""GPU parity of the XCD-split modes against the oracle, teacher-forced at
every layer as in tests/test_gpu_stack.py: the persistent step
(EDGE0_STACK_XCD) and the per-layer launches replayed as graphs
(EDGE0_STACK_XLAYER), on the 40-layer Qwen3-MoE-shaped stack at K = 4 (the
benchmark's configuration) and K = 8, with group biases independent of the
scales, a 6-layer stack of wide layers, switching modes and restarting at
step 0 on one handle, the refused shapes, and a bounded wait forced to time
out from the host."""
import numpy as np
import pytest

from synth import gen as G
from tests.test_gpu_stack import QWEN_CONSUMERS, QWEN_OWNERS, _qwen3_stack, _run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _xcd(ds):
    from int4_expert_streaming_amd import edge0 as E
    ds.stack.set_mode(E.EDGE0_STACK_XCD)
    return E


@pytest.mark.timeout(900)
def test_xcd_stack_qwen3moe_k4_every_layer(torch_cuda):
    S, seed = G.QWEN3_MOE, 0
    ds = _qwen3_stack(S, seed)
    E = _xcd(ds)
    report, rels = _run(ds, S, seed, 4, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xcd] qwen3moe K=4: worst rel-L2 {max(rels):.3e}, median {np.median(rels):.3e}, "
          f"waived {report.count('waived')}/{len(report)}")
    # back to the graph mode and again to the XCD mode on the same handle
    ds.stack.set_mode(E.EDGE0_STACK_GRAPHS)
    _run(ds, S, seed, 2, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    ds.stack.set_mode(E.EDGE0_STACK_XCD)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    ds.stack.close()


@pytest.mark.timeout(900)
def test_xcd_stack_qwen3moe_free_bias(torch_cuda):
    S, seed = G.QWEN3_MOE, 7
    ds = _qwen3_stack(S, seed, free_bias=True)
    E = _xcd(ds)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS,
                        free_bias=True)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xcd] qwen3moe free bias: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


@pytest.mark.timeout(900)
def test_xcd_stack_qwen3moe_k8_every_layer(torch_cuda):
    S, seed = G.QWEN3_MOE.with_k(8), 2
    ds = _qwen3_stack(S, seed)
    E = _xcd(ds)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xcd] qwen3moe K=8: worst rel-L2 {max(rels):.3e}, waived {report.count('waived')}")
    ds.stack.close()


@pytest.mark.timeout(600)
def test_xcd_stack_wide_k8(torch_cuda):
    """d_model 2048, 32 experts, d_inter 384, K = 8, r = 16: one XCD per
    expert, 12 rows per workgroup."""
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S, seed = G.MoEShape(2048, 32, 384, 8, 64, 16, 32.0, 64), 11
    owners, consumers = range(1, 5), range(2, 6)
    ds = DeviceStack(S, G.StackGen(S, seed), 6, (1, 4), (2, 5), log=None)
    E = _xcd(ds)
    report, rels = _run(ds, S, seed, 3, lambda t: range(6), owners, consumers)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xcd] wide K=8: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


def test_xcd_mode_rejects_unsupported_shapes(torch_cuda):
    from int4_expert_streaming_amd import edge0 as E
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    for S in (G.TINY, G.MoEShape(2048, 32, 384, 4, 64, 16, 32.0, 64)):
        ds = DeviceStack(S, G.StackGen(S, 1), 4, (1, 2), (2, 3), log=None)
        with pytest.raises(E.Edge0Error) as ei:
            ds.stack.set_mode(E.EDGE0_STACK_XCD)
        assert ei.value.code == E.EDGE0_EINVAL
        ds.stack.close()


def test_xcd_mode_bounded_wait_reports_error(torch_cuda):
    """A spin limit of one poll: the first hand-off's wait times out in some
    workgroup, which records EDGE0_EHIP and raises the abort word; every
    workgroup then leaves, so the launch ends and reports the error."""
    import torch
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE
    ds = DeviceStack(S, G.StackGen(S, 5), 4, (1, 2), (2, 3), log=None)
    E = _xcd(ds)
    ds.stack.set_spin_limit(1)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    ds.step(to_device(G.stack_hidden(S, 5, 0)), h_out, 0)
    torch.cuda.synchronize()
    assert ds.stack.error() == E.EDGE0_EHIP
    ds.stack.close()


# ---------------------------------------------------------------- XLAYER
def _xlayer(ds):
    from int4_expert_streaming_amd import edge0 as E
    ds.stack.set_mode(E.EDGE0_STACK_XLAYER)
    return E


@pytest.mark.timeout(900)
def test_xlayer_stack_qwen3moe_k4_every_layer(torch_cuda):
    S, seed = G.QWEN3_MOE, 0
    ds = _qwen3_stack(S, seed)
    E = _xlayer(ds)
    report, rels = _run(ds, S, seed, 4, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xlayer] qwen3moe K=4: worst rel-L2 {max(rels):.3e}, median {np.median(rels):.3e}, "
          f"waived {report.count('waived')}/{len(report)}")
    # the graph mode on the same handle, then this mode again from step 0
    ds.stack.set_mode(E.EDGE0_STACK_GRAPHS)
    _run(ds, S, seed, 2, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    ds.stack.set_mode(E.EDGE0_STACK_XLAYER)
    report, rels = _run(ds, S, seed, 8, lambda t: range(40) if t in (0, 1, 6, 7) else [7, 20],
                        QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    ds.stack.close()


@pytest.mark.timeout(900)
def test_xlayer_stack_qwen3moe_free_bias(torch_cuda):
    S, seed = G.QWEN3_MOE, 7
    ds = _qwen3_stack(S, seed, free_bias=True)
    E = _xlayer(ds)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS,
                        free_bias=True)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xlayer] qwen3moe free bias: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


@pytest.mark.timeout(900)
def test_xlayer_stack_qwen3moe_k8_every_layer(torch_cuda):
    S, seed = G.QWEN3_MOE.with_k(8), 2
    ds = _qwen3_stack(S, seed)
    E = _xlayer(ds)
    report, rels = _run(ds, S, seed, 3, lambda t: range(40), QWEN_OWNERS, QWEN_CONSUMERS)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xlayer] qwen3moe K=8: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


@pytest.mark.timeout(600)
def test_xlayer_stack_wide_k8(torch_cuda):
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    S, seed = G.MoEShape(2048, 32, 384, 8, 64, 16, 32.0, 64), 11
    owners, consumers = range(1, 5), range(2, 6)
    ds = DeviceStack(S, G.StackGen(S, seed), 6, (1, 4), (2, 5), log=None)
    E = _xlayer(ds)
    report, rels = _run(ds, S, seed, 4, lambda t: range(6), owners, consumers)
    assert ds.stack.error() == E.EDGE0_OK
    assert report.count("exact") >= 0.8 * len(report), report
    print(f"[xlayer] wide K=8: worst rel-L2 {max(rels):.3e}")
    ds.stack.close()


def test_xlayer_mode_bounded_wait_reports_error(torch_cuda):
    import torch
    from int4_expert_streaming_amd.stackbuild import DeviceStack
    from int4_expert_streaming_amd.weights import to_device
    S = G.QWEN3_MOE
    ds = DeviceStack(S, G.StackGen(S, 5), 4, (1, 2), (2, 3), log=None)
    E = _xlayer(ds)
    ds.stack.set_spin_limit(1)
    h_out = torch.zeros(S.d_model, dtype=torch.int16, device="cuda")
    ds.step(to_device(G.stack_hidden(S, 5, 0)), h_out, 0)
    torch.cuda.synchronize()
    assert ds.stack.error() == E.EDGE0_EHIP
    ds.stack.close()
