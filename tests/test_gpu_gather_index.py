"""The opt-in index check of gather_qmm and the kernel-path query, on the GPU.

"EMLX.Quantization", gather_quantized_matmul: rhs_indices names each row's
expert and lhs_indices its activation batch entry; indices are a
precondition of the library. With QLIN_CHECK_INDICES=1 a small kernel checks
them first and a bad index fails the call before any gather kernel runs.
Only in-range indices ever reach a gather kernel in these tests: every
out-of-range case runs with the check on, where the check kernel (which reads
the index arrays within their bounds) is the only kernel launched.
"""
import os

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

qm = pytest.importorskip("quantized_matmul_amd")

DEV = "cuda:0"
INVALID, UNSUPPORTED = 1, 2


@pytest.fixture(autouse=True)
def _clean_env():
    for k in ("QLIN_FORCE_PATH", "QLIN_CHECK_INDICES"):
        os.environ.pop(k, None)
    yield
    for k in ("QLIN_FORCE_PATH", "QLIN_CHECK_INDICES"):
        os.environ.pop(k, None)


def _problem(T, E, k, N, K, wid):
    w, _ = synth.normal((E, N, K), 0.02, wid, synth.WEIGHT, "bf16")
    x, _ = synth.normal((T, 1, K), 1.0, wid, synth.ACT, "bf16")
    qw = qm.quantize(w.to(DEV), 64, 4)
    rhs = torch.from_numpy(synth.topk_distinct(T, E, k, wid).astype(np.int32)).to(DEV)
    lhs = torch.arange(T, dtype=torch.int32, device=DEV).repeat_interleave(k).reshape(T, k)
    return x.to(DEV), qw, rhs, lhs


# (tokens, experts, top-k): decode-sized (direct and tiled gather forms of the
# small-M kernel) and many rows (bucketing + many-row MFMA kernel)
SHAPES = [(1, 16, 4), (6, 16, 4), (96, 8, 2)]


@pytest.mark.parametrize("T,E,k", SHAPES)
@pytest.mark.parametrize("path", [None, "tiled", "generic"])
def test_check_on_valid_indices_is_bit_identical(T, E, k, path):
    x, qw, rhs, lhs = _problem(T, E, k, 192, 512, 80 + T)
    print(f"index check valid T{T} E{E} k{k} path={path}", flush=True)
    if path:
        os.environ["QLIN_FORCE_PATH"] = path
    y0 = qm.gather_qmm(x, qw, rhs, lhs)
    os.environ["QLIN_CHECK_INDICES"] = "1"
    y1 = qm.gather_qmm(x, qw, rhs, lhs)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("T,E,k", SHAPES)
def test_check_rejects_out_of_range_rhs(T, E, k):
    x, qw, rhs, lhs = _problem(T, E, k, 192, 512, 90 + T)
    bad = rhs.clone().reshape(-1)
    r = bad.numel() // 2
    bad[r] = E                      # one past the last expert
    bad = bad.reshape(rhs.shape)
    y = torch.full((T, k, 1, 192), 7.0, dtype=torch.bfloat16, device=DEV)
    os.environ["QLIN_CHECK_INDICES"] = "1"
    print(f"index check bad rhs row {r} T{T} E{E} k{k}", flush=True)
    with pytest.raises(qm.QlinError) as ei:
        qm.gather_qmm(x, qw, bad, lhs, out=y)
    torch.cuda.synchronize()
    assert ei.value.status == INVALID
    assert f"rhs_indices[{r}] = {E}" in str(ei.value)
    assert torch.all(y == 7.0)      # nothing but the check ran


def test_check_rejects_out_of_range_lhs_and_batch():
    T, E, k = 6, 16, 4
    x, qw, rhs, lhs = _problem(T, E, k, 192, 512, 97)
    bad = lhs.clone().reshape(-1)
    bad[5] = T + 3
    os.environ["QLIN_CHECK_INDICES"] = "1"
    with pytest.raises(qm.QlinError) as ei:
        qm.gather_qmm(x, qw, rhs, bad.reshape(lhs.shape))
    assert ei.value.status == INVALID and f"lhs_indices[5] = {T + 3}" in str(ei.value)
    # the first bad row is the one reported
    bad2 = rhs.clone().reshape(-1)
    bad2[3] = 1000
    bad2[9] = 99
    with pytest.raises(qm.QlinError) as ei:
        qm.gather_qmm(x, qw, bad2.reshape(rhs.shape), lhs)
    assert "rhs_indices[3] = 1000" in str(ei.value)
    torch.cuda.synchronize()


def test_check_refuses_graph_capture():
    T, E, k = 1, 16, 4
    x, qw, rhs, lhs = _problem(T, E, k, 192, 512, 98)
    ws = torch.empty(qm.gather_qmm_workspace_bytes(T * k, E), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, k, 1, 192), dtype=torch.bfloat16, device=DEV)
    qm.gather_qmm(x, qw, rhs, lhs, workspace=ws, out=y)     # warm-up outside the capture
    torch.cuda.synchronize()
    os.environ["QLIN_CHECK_INDICES"] = "1"
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g):
        try:
            qm.gather_qmm(x, qw, rhs, lhs, workspace=ws, out=y)
        except qm.QlinError as e:
            status = e.status
    assert status == UNSUPPORTED
    torch.cuda.synchronize()


def test_last_path_names_the_kernel():
    w, _ = synth.normal((256, 512), 0.02, 99, synth.WEIGHT, "bf16")
    qw = qm.quantize(w.to(DEV), 64, 4)
    x1, _ = synth.normal((1, 512), 1.0, 99, synth.ACT, "bf16")
    qm.quantized_matmul(x1.to(DEV), qw)
    assert qm.last_path() == "decode"
    x2, _ = synth.normal((300, 512), 1.0, 99, synth.ACT, "bf16")
    qm.quantized_matmul(x2.to(DEV), qw)
    assert qm.last_path() == "prefill"
    wf, _ = synth.normal((256, 512), 0.02, 99, synth.WEIGHT, "f32")
    qf = qm.quantize(wf.to(DEV), 64, 4)
    xf, _ = synth.normal((2, 512), 1.0, 99, synth.ACT, "f32")
    qm.quantized_matmul(xf.to(DEV), qf)
    assert qm.last_path() == "generic"
    torch.cuda.synchronize()
