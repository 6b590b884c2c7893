"""The expert-file tier: the layer file format (header fields, records equal
to the bundles, zero padding to 4096-byte records) and the file tier's
refusals (another layer's or another shape's file, a short file, a missing
path).  The staged stacks read from files are in test_gpu_streamed.py."""
import os
import struct

import numpy as np
import pytest

from synth import gen as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def tiny_files(torch_cuda, tmp_path_factory):
    from int4_expert_streaming_amd.stackbuild import HostBundles, write_layer_files
    S = G.TINY
    host = HostBundles(S, G.StackGen(S, 3), 3, log=None)
    d = tmp_path_factory.mktemp("layers")
    return S, host, write_layer_files(host, str(d), S.n_experts)


def test_layer_file_format(tiny_files):
    from int4_expert_streaming_amd import edge0 as E
    S, host, paths = tiny_files
    sh = E.make_shape(S)
    bb = host.bundle_bytes
    rec = E.lib.edge0_layer_file_record_bytes(E.C.byref(sh))
    assert rec % 4096 == 0 and bb <= rec < bb + 4096
    for L, p in enumerate(paths):
        raw = open(p, "rb").read()
        assert len(raw) == 4096 + S.n_experts * rec
        magic, version, layer, n_exp, _, b_bytes, r_bytes = struct.unpack_from("<8s4i2q", raw, 0)
        assert (magic, version, layer, n_exp, b_bytes, r_bytes) == (b"E0LAYER1", 1, L, S.n_experts,
                                                                   bb, rec)
        shape_raw = raw[40:40 + E.C.sizeof(E.MoeShape)]
        assert shape_raw == bytes(sh)
        for e in range(S.n_experts):
            off = 4096 + e * rec
            assert raw[off:off + bb] == host.bundle(L, e, S.n_experts).numpy().tobytes(), (L, e)
            assert raw[off + bb:off + rec] == bytes(rec - bb)


def test_filetier_refuses_mismatched_files(tiny_files, tmp_path):
    from int4_expert_streaming_amd import edge0 as E
    S, host, paths = tiny_files
    sh = E.make_shape(S)
    ft = E.FileTier(sh, paths)  # the right files open
    ft.close()
    bad_sets = [[paths[1], paths[0], paths[2]],          # layer 0 given layer 1's file
                [paths[0], str(tmp_path / "none"), paths[2]]]
    short = tmp_path / "short.e0l"
    short.write_bytes(open(paths[2], "rb").read()[:-4096])
    bad_sets.append([paths[0], paths[1], str(short)])
    for ps in bad_sets:
        with pytest.raises(E.Edge0Error) as ei:
            E.FileTier(sh, ps)
        assert ei.value.code == E.EDGE0_EINVAL
    other = E.make_shape(G.TINY)
    other.lora_alpha = 8.0  # another shape than the files were written for
    with pytest.raises(E.Edge0Error):
        E.FileTier(other, paths)
    with pytest.raises(E.Edge0Error):
        E.FileTier(sh, paths, n_buffers=8)  # fewer buffers than one request may miss
