"""The allocation-free gather entry point (qlin_gather_qmm_noalloc) against
qlin_gather_qmm with a caller's workspace, through the C ABI.

Both run the same kernels, so every output must be bit-identical. Two calls
in a row on the library's shared scratch, the second smaller than the first
(the scratch keeps the first call's contents), then a third at the first
size again, each checked against the workspace entry point; the noalloc
call also runs inside a HIP graph capture and on replays.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

qm = pytest.importorskip("quantized_matmul_amd")

DEV = "cuda:0"


def _case(T, E, k, N, K, wid, mode="affine", g=64, bits=4):
    w, _ = synth.normal((E, N, K), 0.02, wid, synth.WEIGHT, "bf16")
    x, _ = synth.normal((T, 1, K), 1.0, wid, synth.ACT, "bf16")
    qw = qm.quantize(w.to(DEV), g, bits, mode)
    rhs = torch.from_numpy(synth.topk_distinct(T, E, k, wid).astype(np.int32)).to(DEV)
    lhs = torch.arange(T, dtype=torch.int32, device=DEV).repeat_interleave(k).reshape(T, k)
    return x.to(DEV), qw, rhs.contiguous(), lhs.contiguous()


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("sorted_indices", [False, True])
def test_noalloc_matches_workspace_entry_point(sorted_indices):
    # 256 tokens x top-4 of 32 experts (bucketing + many-row kernel), then
    # smaller decode-sized calls (20 tokens: bucketed 16-row tiles; 2 tokens:
    # one tile per index row), then the large one again
    cases = [(256, 32, 4, 384, 1024, 110), (20, 32, 4, 384, 1024, 111), (2, 32, 4, 384, 1024, 112),
             (256, 32, 4, 384, 1024, 113)]
    for T, E, k, N, K, wid in cases:
        x, qw, rhs, lhs = _case(T, E, k, N, K, wid)
        if sorted_indices:
            order = torch.argsort(rhs.reshape(-1), stable=True)
            rhs = rhs.reshape(-1)[order].contiguous()
            lhs = lhs.reshape(-1)[order].contiguous()
        print(f"noalloc T{T} E{E} k{k} N{N} K{K} sorted={sorted_indices}", flush=True)
        y_ref = qm.gather_qmm(x, qw, rhs, lhs, sorted_indices=sorted_indices)
        y = torch.full_like(y_ref, 3.0)
        qm.gather_qmm_noalloc(x, qw, rhs, lhs, sorted_indices=sorted_indices, out=y)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref)), (T, E, k)


def test_noalloc_microscaled_and_many_rows_per_token():
    x, qw, rhs, lhs = _case(64, 16, 2, 256, 512, 120, mode="mxfp4", g=32, bits=4)
    y_ref = qm.gather_qmm(x, qw, rhs, lhs)
    y = qm.gather_qmm_noalloc(x, qw, rhs, lhs)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    x2, qw2, rhs2, lhs2 = _case(3, 16, 2, 256, 512, 114, mode="mxfp4", g=32, bits=4)
    y2 = qm.gather_qmm_noalloc(x2, qw2, rhs2, lhs2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y2), _bits(qm.gather_qmm(x2, qw2, rhs2, lhs2)))


def test_noalloc_under_graph_capture():
    x, qw, rhs, lhs = _case(128, 16, 4, 256, 512, 115)
    y_ref = qm.gather_qmm(x, qw, rhs, lhs)
    y = torch.zeros_like(y_ref)
    qm.gather_qmm_noalloc(x, qw, rhs, lhs, out=y)      # first call on the device: scratch lookup
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qm.gather_qmm_noalloc(x, qw, rhs, lhs, out=y)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref)), rep
        # eager work on the same scratch between replays (a smaller problem)
        xs, qws, rhss, lhss = _case(2, 16, 4, 256, 512, 116 + rep)
        ys = qm.gather_qmm_noalloc(xs, qws, rhss, lhss)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ys), _bits(qm.gather_qmm(xs, qws, rhss, lhss)))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = qm.load_library()
    assert lib.qlin_gather_qmm_noalloc_max_rows() == 65536
    assert lib.qlin_gather_qmm_noalloc_max_experts() == 4096
    x, qw, rhs, lhs = _case(2, 16, 4, 256, 512, 119)
    big_e = ctypes.c_int64(4097)
    vp = ctypes.c_void_p
    rc = lib.qlin_gather_qmm_noalloc(vp(x.data_ptr()), 2, 2, 1, 512, vp(qw.value.data_ptr()),
                                     vp(qw.scales.data_ptr()), vp(qw.biases.data_ptr()), 2, big_e,
                                     256, None, vp(rhs.data_ptr()), 65537, 1, 64, 4, b"affine", 0,
                                     vp(x.data_ptr()), None)
    assert rc == 1
    assert b"at most 65536" in lib.qlin_last_error()
